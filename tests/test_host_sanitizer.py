"""The C ABI layer's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  api.hip and the host sizing code (sizing.hip) are compiled for the host alone,
linked with stand-in launchers (tests/host_check/stubs.cpp) and driven by
tests/host_check/validate_main.cpp: invalid, unsupported, extreme (INT_MAX / INT64_MAX
sizes, products past 64 bits) and valid arguments for every entry point.  A rejected call
must return its status without reaching a launcher, an accepted one must reach exactly one
launcher, and the sanitizers must report nothing (any report aborts the run)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "online_softmax_attn_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "host_check")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

# sanitizers on the host pass only (this build has no device pass at all)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs hipcc and the ROCm clang++ on this host")
def test_abi_validation_under_sanitizers(tmp_path):
    srcs = [os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "sizing.hip"),
            os.path.join(CHECK, "stubs.cpp"), os.path.join(CHECK, "validate_main.cpp")]
    objs = []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "--cuda-host-only", "-x", "hip", "-std=c++17", "-O1", "-g", *SAN,
               f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{CHECK}", "-c", src,
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "host_check")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "0 failures" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
