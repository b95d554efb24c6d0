"""The C ABI: library loads, exports what include/attn.h declares, and rejects bad
host-visible arguments before touching the GPU (CPU only: every call here fails validation
and returns before any HIP call)."""

import ctypes
import os
import re

import pytest

import online_softmax_attn_amd as attn
from online_softmax_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x10000  # a non-null pointer value: validation fails before it could be used
INVALID, UNSUPPORTED, WORKSPACE = (binding.ATTN_ERR_INVALID, binding.ATTN_ERR_UNSUPPORTED,
                                   binding.ATTN_ERR_WORKSPACE)


PROBE_HEADER = os.path.join(ROOT, "include", "attn_probe.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(binding.SIGNATURES), names
    lib = attn.lib()
    for name in names:
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_library_exports_every_probe_function():
    names = declared_functions(PROBE_HEADER)
    assert set(names) == set(binding.PROBE_SIGNATURES), names
    lib = attn.lib()
    for name in names:
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


@pytest.mark.parametrize("call", [
    lambda L: L.attn_probe_mfma(0, 1, 1, None, None),
    lambda L: L.attn_probe_mfma(2, 1, 1, FAKE, None),
    lambda L: L.attn_probe_mfma(0, 0, 1, FAKE, None),
    lambda L: L.attn_probe_mfma(1, 1, 0, FAKE, None),
    lambda L: L.attn_probe_mfma(0, 1, 16385, FAKE, None),
    lambda L: L.attn_probe_exp(0, 1, FAKE, None),
    lambda L: L.attn_probe_exp(1, -1, FAKE, None),
    lambda L: L.attn_probe_exp(1, 1, None, None),
    lambda L: L.attn_probe_read(None, 4096, 1, FAKE, None),
    lambda L: L.attn_probe_read(FAKE, 0, 1, FAKE, None),
    lambda L: L.attn_probe_read(FAKE, 4100, 1, FAKE, None),
    lambda L: L.attn_probe_read(FAKE, 4096, 0, FAKE, None),
    lambda L: L.attn_probe_read_pages(FAKE, 8, None, 8, 1, FAKE, None),
    lambda L: L.attn_probe_read_pages(FAKE, 0, FAKE, 8, 1, FAKE, None),
    lambda L: L.attn_probe_read_pages(FAKE, 8, FAKE, 0, 1, FAKE, None),
    lambda L: L.attn_probe_read_pages(None, 8, FAKE, 8, 1, FAKE, None),
    lambda L: L.attn_probe_mfma(0, (1 << 24) + 1, 1, FAKE, None),
    lambda L: L.attn_probe_exp((1 << 24) + 1, 1, FAKE, None),
    lambda L: L.attn_probe_read(FAKE, 4096, (1 << 24) + 1, FAKE, None),
    lambda L: L.attn_probe_read_pages(FAKE, 8, FAKE, 8, (1 << 24) + 1, FAKE, None),
])
def test_probe_validation(call):
    assert call(attn.lib()) == INVALID


def test_abi_version_matches_header():
    text = open(HEADER).read()
    want = int(re.search(r"#define ATTN_ABI_VERSION (\d+)", text).group(1))
    assert attn.attn_abi_version() == want


def test_status_strings():
    assert attn.attn_status_str(0) == "ATTN_OK"
    assert attn.attn_status_str(UNSUPPORTED) == "ATTN_ERR_UNSUPPORTED"
    assert attn.attn_status_str(99) == "ATTN_ERR_UNKNOWN"


def fwd(**kw):
    a = dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, lens=None, B=1, H=1, Hkv=1,
             n=16, d=128, causal=0, window=0, scale=0.1)
    a.update(kw)
    return attn.lib().attn_fwd(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["lens"],
                               a["B"], a["H"], a["Hkv"], a["n"], a["d"], a["causal"], a["window"],
                               a["scale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID), (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(n=0), INVALID),
    (dict(d=0), INVALID), (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(dtype=0, d=96), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED), (dict(n=1 << 24, d=128), UNSUPPORTED),
    (dict(Hkv=0), INVALID), (dict(H=4, Hkv=3), INVALID), (dict(H=4, Hkv=8), INVALID),
    (dict(window=-1, causal=1), INVALID), (dict(window=8, causal=0), INVALID),
    (dict(H=4, Hkv=2, window=8, causal=1, d=96), UNSUPPORTED),
])
def test_fwd_validation(kw, status):
    assert fwd(**kw) == status


def dec(**kw):
    a = dict(dtype=1, q=FAKE, kc=FAKE, vc=FAKE, tbl=FAKE, lens=FAKE, o=FAKE, lse=None, B=2, H=4,
             Hkv=4, d=128, bs=16, nb=10, mb=8, msl=128, window=0, scale=0.1, split=0, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return attn.lib().attn_decode_paged(a["dtype"], a["q"], a["kc"], a["vc"], a["tbl"], a["lens"],
                                        a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["d"], a["bs"],
                                        a["nb"], a["mb"], a["msl"], a["window"], a["scale"],
                                        a["split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(tbl=None), INVALID),
    (dict(lens=None), INVALID), (dict(o=None), INVALID), (dict(B=0), INVALID),
    (dict(nb=0), INVALID), (dict(msl=0), INVALID), (dict(scale=0.0), INVALID),
    (dict(mb=7), INVALID),               # 7 blocks of 16 cannot hold 128 tokens
    (dict(split=24), INVALID), (dict(split=-16), INVALID), (dict(split=2048), INVALID),
    (dict(bs=32, mb=4), UNSUPPORTED), (dict(d=64), UNSUPPORTED), (dict(dtype=0), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE),
    (dict(Hkv=0), INVALID), (dict(Hkv=3), INVALID), (dict(window=-5), INVALID),
])
def test_decode_validation(kw, status):
    assert dec(**kw) == status


def bwd(**kw):
    a = dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, lens=None, dq=FAKE, dk=FAKE,
             dv=FAKE, B=1, H=1, Hkv=1, n=16, d=128, causal=0, window=0, scale=0.1, ws=FAKE,
             wsb=1 << 20)
    a.update(kw)
    return attn.lib().attn_bwd(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"],
                               a["lens"], a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["Hkv"],
                               a["n"], a["d"], a["causal"], a["window"], a["scale"], a["ws"],
                               a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(do=None), INVALID),
    (dict(lse=None), INVALID), (dict(dq=None), INVALID), (dict(dv=None), INVALID),
    (dict(n=0), INVALID), (dict(scale=float("nan")), INVALID), (dict(d=64), UNSUPPORTED),
    (dict(dtype=0), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(wsb=63), WORKSPACE),
    (dict(H=2, Hkv=4), INVALID), (dict(window=4), INVALID), (dict(window=-1, causal=1), INVALID),
])
def test_bwd_validation(kw, status):
    assert bwd(**kw) == status


def test_bwd_workspace_bytes():
    assert attn.attn_bwd_workspace_bytes(2, 3, 100) == 2 * 3 * 100 * 4
    assert attn.attn_bwd_workspace_bytes(0, 3, 100) == 0


def test_decode_workspace_bytes():
    f = attn.attn_decode_workspace_bytes
    # partials: B * H * ceil(max_seq_len / split) entries of (m, l, u[128]) fp32
    assert f(2, 4, 128, 1000, 256) == 2 * 4 * 4 * 130 * 4
    assert f(2, 4, 128, 1024, 16) == 2 * 4 * 64 * 130 * 4
    assert f(2, 4, 128, 1000, 0) > 0
    assert f(2, 4, 64, 1000, 0) == 0
    assert f(2, 4, 128, 1000, 24) == 0
    assert f(0, 4, 128, 1000, 0) == 0
    need = f(2, 4, 128, 128, 0)
    assert dec(wsb=need - 1) == WORKSPACE
    # a window of w tokens touches at most ceil((w + 15) / 16) blocks: 300 -> 19 blocks,
    # 2 splits of 256 tokens instead of 4 for the whole 1000
    assert f(2, 4, 128, 1000, 256, window=300) == 2 * 4 * 2 * 130 * 4
    assert f(2, 4, 128, 1000, 256, window=5000) == f(2, 4, 128, 1000, 256)
    assert f(2, 4, 128, 1000, 256, kv_heads=3) == 0
    assert f(2, 4, 128, 1000, 256, window=-1) == 0
    need = f(2, 4, 128, 128, 0, kv_heads=2, window=40)
    assert need > 0 and dec(Hkv=2, window=40, wsb=need - 1) == WORKSPACE


def q8(**kw):
    a = dict(x=FAKE, x8=FAKE, sc=FAKE, lens=None, B=1, H=2, n=100, d=128, tr=0)
    a.update(kw)
    return attn.lib().attn_quantize_fp8(a["x"], a["x8"], a["sc"], a["lens"], a["B"], a["H"], a["n"],
                                        a["d"], a["tr"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(x8=None), INVALID), (dict(sc=None), INVALID),
    (dict(B=0), INVALID), (dict(n=-1), INVALID), (dict(d=64), UNSUPPORTED),
    (dict(B=300, H=300), UNSUPPORTED),
])
def test_quantize_fp8_validation(kw, status):
    assert q8(**kw) == status


def f8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sq=FAKE, sk=FAKE, sv=FAKE, o=FAKE, lse=None, lens=None, B=1,
             H=4, Hkv=2, n=100, d=128, causal=1, scale=0.1)
    a.update(kw)
    return attn.lib().attn_fwd_fp8(a["q"], a["k"], a["v"], a["sq"], a["sk"], a["sv"], a["o"],
                                   a["lse"], a["lens"], a["B"], a["H"], a["Hkv"], a["n"], a["d"],
                                   a["causal"], a["scale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(v=None), INVALID), (dict(sk=None), INVALID), (dict(o=None), INVALID),
    (dict(H=0), INVALID), (dict(Hkv=3), INVALID), (dict(scale=-1.0), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(n=1 << 24), UNSUPPORTED),
])
def test_fwd_fp8_validation(kw, status):
    assert f8(**kw) == status


def mg(**kw):
    a = dict(dt=attn.ATTN_BF16, parts=FAKE, lses=FAKE, o=FAKE, lse=None, S=4, rows=1000, d=128)
    a.update(kw)
    return attn.lib().attn_merge(a["dt"], a["parts"], a["lses"], a["o"], a["lse"], a["S"], a["rows"],
                                 a["d"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(parts=None), INVALID), (dict(lses=None), INVALID), (dict(o=None), INVALID),
    (dict(S=0), INVALID), (dict(rows=0), INVALID), (dict(rows=-5), INVALID), (dict(d=0), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(dt=7), UNSUPPORTED), (dict(S=1025), UNSUPPORTED),
    (dict(rows=1 << 36), UNSUPPORTED),
])
def test_merge_validation(kw, status):
    assert mg(**kw) == status


def ch(**kw):
    a = dict(dt=attn.ATTN_BF16, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H=4, Hkv=2,
             nq=100, nkv=300, q0=200, d=128, causal=1, window=0, scale=0.1)
    a.update(kw)
    return attn.lib().attn_fwd_chunk(a["dt"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                     a["H"], a["Hkv"], a["nq"], a["nkv"], a["q0"], a["d"],
                                     a["causal"], a["window"], a["scale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID), (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(nq=0), INVALID),
    (dict(nkv=0), INVALID), (dict(d=0), INVALID), (dict(q0=-1), INVALID),
    (dict(q0=201), INVALID), (dict(nq=301, q0=0), INVALID), (dict(Hkv=0), INVALID),
    (dict(H=4, Hkv=3), INVALID), (dict(window=-1), INVALID), (dict(window=8, causal=0), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(dt=attn.ATTN_F32), UNSUPPORTED), (dict(dt=7), UNSUPPORTED), (dict(d=32), UNSUPPORTED),
    (dict(nkv=1 << 24, nq=16, q0=0), UNSUPPORTED),
])
def test_fwd_chunk_validation(kw, status):
    assert ch(**kw) == status


def dec_noalloc(**kw):
    a = dict(dtype=1, q=FAKE, kc=FAKE, vc=FAKE, tbl=FAKE, lens=FAKE, o=FAKE, lse=None, B=2, H=4,
             Hkv=4, d=128, bs=16, nb=16, mb=8, msl=128, window=0, scale=0.1, split=0)
    a.update(kw)
    return attn.lib().attn_decode_paged_noalloc(
        a["dtype"], a["q"], a["kc"], a["vc"], a["tbl"], a["lens"], a["o"], a["lse"], a["B"],
        a["H"], a["Hkv"], a["d"], a["bs"], a["nb"], a["mb"], a["msl"], a["window"], a["scale"],
        a["split"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(lens=None), INVALID),
    (dict(B=0), INVALID), (dict(mb=7), INVALID), (dict(split=24), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(bs=32, mb=4), UNSUPPORTED), (dict(Hkv=3), INVALID),
    # partials past the fixed scratch array: 64 x 64 heads x 128 splits of 520 bytes
    (dict(B=64, H=64, Hkv=64, msl=65536, mb=4096, split=512), WORKSPACE),
])
def test_decode_noalloc_validation(kw, status):
    """The no-alloc decode runs every check of attn_decode_paged, and refuses partials that
    would not fit its scratch array, before any HIP call."""
    assert dec_noalloc(**kw) == status


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert attn.ATTN_NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
