"""Host-side pieces of bench.py, on the CPU: the algorithmic flop and byte counts it divides
by, the scaling of the HBM traffic counters, and the one-GPU guard."""

import csv
import json
import math
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _pairs(n, window):
    """Admitted (query, key) pairs of causal attention over n tokens, counted one by one."""
    return sum(1 for i in range(n) for j in range(i + 1) if not window or j > i - window)


@pytest.mark.parametrize("n", [1, 7, 64, 130])
@pytest.mark.parametrize("window", [0, 1, 5, 200])
def test_causal_flops_counts_the_admitted_pairs(n, window):
    B, H, d = 2, 3, 128
    assert bench.causal_flops(B, H, n, d, window) == 4.0 * d * B * H * _pairs(n, window)


def test_causal_flops_of_the_causal_prefill_workload():
    # [4, 32, 2048, 128]: 4 d flops (Q K^T and P V) per admitted pair, 2048 * 2049 / 2 pairs
    assert bench.causal_flops(4, 32, 2048, 128) == pytest.approx(1.3751e11, rel=1e-4)


@pytest.mark.parametrize("window", [0, 20])
def test_decode_bytes_counts_admitted_tokens_query_output_and_table(window):
    lens = [1, 17, 40]
    w = workloads.paged(lens, 4, 128, seed=5, kv_heads=2)
    kv = sum(min(L, window) if window else L for L in lens) * 2 * 128 * 2 * 2  # K and V, bf16
    q_o = 2 * 3 * 4 * 128 * 2                                                    # q and o, bf16
    table = 4 * sum(math.ceil(L / 16) - (max(L - window, 0) // 16 if window else 0) for L in lens)
    assert bench.decode_bytes(w, 2, 128, window) == kv + q_o + table


def _counter_csv(path, counter, values):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, kib) in enumerate(values):
            wr.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": kib})


def test_record_traffic_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kernels = ["__amd_rocclr_copyBuffer", "fwd_bf16_kernel<false>", "decode_split_kernel<1>",
               "decode_merge_kernel"]
    # the 1 GiB copy reads as 0.5 GiB of FETCH_SIZE and 1 GiB of WRITE_SIZE (KiB)
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", zip(kernels, [524288, 1000, 3000, 10]))
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", zip(kernels, [1048576, 64, 5, 1]))
    bench.record_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = json.load(open(tmp_path / "traffic.json"))
    assert rec["scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    assert rec["prefill"]["fetch_bytes"] == 1000 * 1024 * 2
    assert rec["prefill"]["write_bytes"] == 64 * 1024
    assert rec["prefill"]["bytes_per_launch"] == (2000 + 64) * 1024
    assert rec["decode"]["bytes_per_launch"] == (3000 * 2 + 5 + 10 * 2 + 1) * 1024
    assert rec["prefill"]["kernel_hash"] == bench.kernel_hash(bench.KERNEL_FILES["prefill"])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_summarize_trace_averages_exactly_the_timed_launches(tmp_path, capsys):
    # launch order: 3 untimed prefills, then K = 2 timed ones; long and decode likewise
    rows, t = [], 0
    def add(name, grid, dur):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur,
                     "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
        t += dur + 10
    for dur in (900, 800, 700, 150_000, 170_000):           # ns; the last two are timed
        add("void fwd_bf16_kernel<false>(...)", 2048 * 256, dur)
    for dur in (9_000_000, 8_000_000, 8_200_000):          # first long launch is untimed
        add("void fwd_bf16_kernel<false>(...)", 8192 * 256, dur)
    for dur in (400_000, 380_000, 390_000):
        add("void decode_split_kernel<1>(...)", 32 * 32 * 16 * 64, dur)
        add("void decode_merge_kernel(...)", 32 * 32 * 64, 5_000)
    with open(tmp_path / "trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)
    line = {"metric": "m", "steps": 2, "prefill": {"ms_avg": 0.16}, "long_prefill": {"ms_avg": 8.1},
            "decode": {"ms_avg": 0.39},
            "trace_index": {"prefill_first": 3, "long_first": 1, "decode_first": 1}}
    (tmp_path / "line.log").write_text("noise\n" + json.dumps(line) + "\n")
    bench.summarize_trace(str(tmp_path / "trace.csv"), str(tmp_path / "line.log"))
    out = capsys.readouterr().out
    assert "| 160.00 | 160.00 |" in out          # (150 + 170) / 2 us, line 0.16 ms
    assert "| 8100.00 | 8100.00 |" in out        # (8000 + 8200) / 2 us
    assert "| 390.00 |" in out                   # decode split + merge: (380+390)/2 + 5


def test_summarize_trace_legs_takes_the_indexed_launches(tmp_path, capsys):
    # one kernel name shared by two timed groups (tags), with untimed launches before each
    rows, t = [], 0
    for name, dur in [("void decode_gqa_kernel(...)", 1_000)] * 2 + \
                     [("void decode_gqa_kernel(...)", 100_000), ("void decode_gqa_kernel(...)", 120_000),
                      ("void decode_gqa_kernel(...)", 200_000), ("void decode_gqa_kernel(...)", 220_000),
                      ("void bwd_dq_kernel(...)", 50_000)]:
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 10
    with open(tmp_path / "trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)
    line = {"metric": "m", "steps": 2,
            "trace_index": {"decode_gqa_kernel#H32": [2, 2], "decode_gqa_kernel#H64": [4, 2],
                            "bwd_dq_kernel": [0, 1]}}
    (tmp_path / "line.log").write_text(json.dumps(line) + "\n")
    bench.summarize_trace(str(tmp_path / "trace.csv"), str(tmp_path / "line.log"))
    out = capsys.readouterr().out
    assert "| decode_gqa_kernel#H32 | 6 | 2 | 110.00 |" in out
    assert "| decode_gqa_kernel#H64 | 6 | 2 | 210.00 |" in out
    assert "| bwd_dq_kernel | 1 | 1 | 50.00 |" in out
