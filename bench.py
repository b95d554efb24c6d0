"""Benchmark of the attention hot path on one MI355X.

Default run (`python bench.py`): one step is one pass of the hot path over the three bf16
workloads that fit one GPU, inputs generated on the host from fixed seeds and moved to HBM
before anything is timed:
  * causal prefill [4, 32, 2048, 128] (attn_fwd)                                   -> `value`
  * paged decode of 32 sequences x 32 heads, d = 128, KV lengths U{1024..8192} in
    16-token pages (attn_decode_paged), each call after a 1 GiB scratch write so that no
    call finds the cache in the 256 MB MALL                                        -> `decode`
  * long-context causal prefill [1, 32, 32768, 128] (attn_fwd)                     -> `long_prefill`

Order of work:
  1. settle: the three legs run round-robin for a fixed wall time (`settle.ms`, default
     400 ms; the shader clock takes tens of ms of sustained load to ramp up), independent
     of --warmup;
  2. W untimed warm-up steps;
  3. the K timed steps, bracketed by synchronisations: K causal prefills back to back
     between one pair of HIP events (an event between two kernels would add the next one's
     dispatch latency to every launch); K flushed decodes, each between its own event pair;
     K long prefills back to back between one event pair.  `value`, `decode.value` and
     `long_prefill.tflops` are the averages over these K launches;
  4. per-launch statistics (median and min): 50 bursts of 5 back-to-back causal prefills
     (per-launch time = burst time / 5), 50 flushed decodes, 50 long prefills; the decode
     back to back (no flush) and the causal prefill with cold caches (inputs cycled over
     600 MB of copies) for reference;
  5. the CPU-baseline leg: the fp64 oracle timed on this host's cores over (batch, head)
     pairs of the causal prefill (bounded to ~12 s), and the parity of this run's GPU
     outputs against the oracle (`parity`: causal prefill on the pairs the oracle
     evaluated, the whole decode, 64 seeded rows per head of the long prefill), each with
     the bf16 output-rounding floor max|bf16(o_ref) - o_ref|.

FLOP/s count algorithmic work only: 4 d flops (QK^T and PV) per admitted causal pair.
Decode GB/s count the admitted K/V tokens, the query, the output and the block-table
entries read.  `roofline` describes the causal prefill kernel against the bf16 dense MFMA
peak; `decode.roofline` the decode against HBM.  `env` records versions, the device, the
host cores this process may run on, and the GPU clock sampled during the timed steps.

--workload long | grouped | window | fp8 | backward | cp | cp-ring | shapes | ceilings
                  other legs (settled and timed the same way, one JSON line each):
  long      the [1, 32, 32768, 128] causal prefill alone;
  grouped   causal prefill and decode with 8 K/V heads for the 32 query heads, and the
            same cache decoded for 64 and 128 query heads (groups of 8 and 16);
  window    causal window 1024: prefill [1, 32, 16384, 128], decode of the decode workload;
  fp8       causal prefill [4, 32, 2048, 128] on E4M3 operands (attn_fwd_fp8), the block
            quantisation (attn_quantize_fp8) timed apart; roofline: dense fp8 MFMA peak;
  backward  attn_bwd on [4, 32, 2048, 128] causal (2.5x the forward's flops);
  cp        one device's share of sequence-parallel causal attention over [1,32,32768,128]
            (16 chunks for 8 devices, zig-zag; device 0): one attn_fwd_chunk per owned
            query chunk against the gathered K/V;
  cp-ring   the same share as a ring delivers K/V chunks: attn_fwd per chunk pair, then
            attn_merge;
  shapes    throughput across shapes (prefill, fp32, fp8, backward, decode), one JSON line
            per shape, under sustained load;
  ceilings  the device's own ceilings from the library's probe kernels (include/attn_probe.h):
            dense bf16 and fp8 MFMA rate, v_exp_f32 rate, HBM read bandwidth streamed and in
            4 KiB pages in random order, each with its checksum verified.
--profile-pass    one 1 GiB device copy, one causal prefill and one decode, then exit (the
                  command the rocprofv3 counter runs wrap).
--profile-pass long
                  30 long-context prefills back to back, then exit (counters of the long
                  prefill under sustained load).
--record-traffic FETCH_CSV WRITE_CSV
                  reads the counter_collection.csv of a FETCH_SIZE and of a WRITE_SIZE run
                  of --profile-pass, scales each counter by what it read for the 1 GiB
                  copy, writes profiles/traffic.json (bytes per launch + kernel hash).
--summarize-trace KERNEL_TRACE_CSV BENCH_JSON_LINE_FILE
                  per-kernel durations of a rocprofv3 kernel trace of a default run, and
                  the average over exactly the launches the run's timed steps covered,
                  next to the line's own figures.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_FP64_TFLOPS = 78.6     # MI355X fp64 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FLUSH_BYTES = 1 << 30       # scratch written before each flushed decode (4x the MALL)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "online_softmax_attn_amd", "csrc")
METRIC = "attn fwd TFLOPS (causal bf16 prefill) + paged-decode HBM GB/s, % of MI355X peak"


def kernel_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_FILES = {"prefill": ["fwd_bf16.hip", "common.h"], "decode": ["decode.hip", "common.h"]}


def recorded_traffic(kind):
    """HBM bytes per launch from the committed counter runs, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_hash") != kernel_hash(KERNEL_FILES[kind]):
        return None
    return rec.get("bytes_per_launch")


def causal_flops(B, H, n, d, window=0):
    """4 d flops (QK^T and PV) per admitted pair; a window admits min(i + 1, w) keys."""
    if not window or window >= n:
        return 4.0 * d * B * H * n * (n + 1) / 2
    pairs = window * (window + 1) / 2 + (n - window) * window
    return 4.0 * d * B * H * pairs


def decode_bytes(w, H_kv, d, window=0):
    """Admitted K/V tokens of every K/V head, the query and output, the table entries read."""
    bs = w.block_size
    kv = q_o = table = 0
    for L in (int(x) for x in w.seq_lens):
        lo = max(L - window, 0) if window else 0
        kv += (L - lo) * H_kv * d * 2 * 2
        table += (math.ceil(L / bs) - lo // bs) * 4
    q_o = 2 * w.q.numel() * 2
    return kv + q_o + table


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# --------------------------------------------------------------------------- timing helpers
class ClockSampler:
    """GPU shader-clock (MHz) and socket-power (W) readings polled every ~5 ms on a side
    thread while phases run; `mark(name)` labels what runs from then on.  The source is the
    SMI library's GPU metrics table (mean of the per-XCD current GFX clocks, current socket
    power), read through the handle torch keeps for it.  The firmware refreshes that table
    about once per second, so only the readings with a new firmware timestamp are kept:
    each is the state at one refresh, and a phase shorter than a second may hold none."""

    def __init__(self):
        self.samples = []          # (phase, t, MHz, W)
        self.phase = "idle"
        self.error = None
        self._stop = threading.Event()
        self._t = None
        self._read = None

    def _reader(self):
        import amdsmi
        import torch

        handle = torch.cuda._get_amdsmi_handler(0)

        def read():
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            ts = m.get("firmware_timestamp")
            w = m.get("current_socket_power")
            w = float(w) if isinstance(w, (int, float)) else 0.0
            xs = [x for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and 0 < x < 10000]
            if xs:
                return sum(xs) / len(xs), w, ts
            x = m.get("current_gfxclk")
            return (float(x) if isinstance(x, (int, float)) else 0.0), w, ts

        read()
        return read

    def start(self):
        try:
            self._read = self._reader()
        except Exception as e:  # no SMI access: the line says so
            self.error = f"{type(e).__name__}: {e}"[:200]
            return self

        def run():
            t0 = time.perf_counter()
            last = None
            while not self._stop.is_set():
                try:
                    mhz, watts, ts = self._read()
                except Exception as e:
                    self.error = f"{type(e).__name__}: {e}"[:200]
                    return
                if ts != last:  # a refresh of the table
                    last = ts
                    self.samples.append((self.phase, time.perf_counter() - t0, float(mhz), watts))
                self._stop.wait(0.005)

        self._t = threading.Thread(target=run, daemon=True)
        self._t.start()
        return self

    def mark(self, phase):
        self.phase = phase

    def stop(self):
        self._stop.set()
        if self._t:
            self._t.join(timeout=2)

    def summary(self, phases):
        vals = [m for p, _, m, _ in self.samples if p in phases and m > 0]
        watts = [w for p, _, m, w in self.samples if p in phases and m > 0 and w > 0]
        out = {"source": "amdsmi GPU metrics, mean of the per-XCD current GFX clocks and the "
                         "current socket power, one reading per refresh of the table (about "
                         "once per second)",
               "phases": sorted(phases), "readings": len(vals)}
        if vals:
            out.update(median_mhz=round(statistics.median(vals), 1), min_mhz=round(min(vals), 1),
                       max_mhz=round(max(vals), 1))
        if watts:
            out.update(median_w=round(statistics.median(watts), 1), min_w=round(min(watts), 1),
                       max_w=round(max(watts), 1))
        if self.error:
            out["error"] = self.error
        return out


def settle(fns, seconds):
    """Run the launches round-robin for `seconds` of wall time; returns (ms, rounds)."""
    import torch

    t0 = time.perf_counter()
    rounds = 0
    while time.perf_counter() - t0 < seconds:
        for f in fns:
            f()
        rounds += 1
        if rounds % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3, rounds


def events(n):
    import torch

    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def burst_ms(fn, reps):
    """Average ms per launch over `reps` back-to-back launches between one event pair (one
    untimed launch first keeps the GPU busy while the burst is enqueued)."""
    import torch

    a, b = events(2)
    fn()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def burst_stats(fn, bursts=50, per=5):
    """Per-launch times from `bursts` bursts of `per` back-to-back launches."""
    import torch

    evs = events(bursts + 1)
    fn()
    evs[0].record()
    for i in range(bursts):
        for _ in range(per):
            fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = [evs[i].elapsed_time(evs[i + 1]) / per for i in range(bursts)]
    return stats(ms, f"{bursts} bursts of {per} back-to-back launches (burst time / {per})")


def flushed_times(fn, flush, reps):
    """ms of each of `reps` launches, each after `flush()` and between its own event pair."""
    import torch

    evs = events(2 * reps)
    for i in range(reps):
        flush()
        evs[2 * i].record()
        fn()
        evs[2 * i + 1].record()
    torch.cuda.synchronize()
    return [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(reps)]


def stats(ms, how):
    return {"reps": len(ms), "how": how, "median_ms": round(statistics.median(ms), 5),
            "min_ms": round(min(ms), 5), "max_ms": round(max(ms), 5)}


def flops_rate(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def roofline_mfma(tflops, peak=PEAK_BF16_TFLOPS, traffic=None):
    return {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4), "traffic": traffic}


def roofline_hbm(gbs, traffic=None):
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}


def env_info():
    import torch

    info = {"torch": torch.__version__, "hip_runtime": getattr(torch.version, "hip", None),
            "affinity_cores": host_cores()}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    try:
        r = subprocess.run(["hipcc", "--version"], capture_output=True, text=True, timeout=30)
        line = next((x for x in r.stdout.splitlines() if "clang version" in x), "")
        info["hipcc"] = line.strip() or None
    except (OSError, subprocess.SubprocessError):
        info["hipcc"] = None
    p = torch.cuda.get_device_properties(0)
    info["device"] = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
                      "compute_units": p.multi_processor_count,
                      "memory_gib": round(p.total_memory / 2**30, 1)}
    return info


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(q, k, v, budget_s=12.0):
    """The oracle as it stands, timed on (batch, head) pairs of the causal prefill until
    ~budget_s has elapsed.  Returns (line entry, {(b, h): oracle output})."""
    import threadpoolctl

    import oracle

    B, H, n, d = q.shape
    outs = {}
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(H):
            o, _ = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                    causal=True)
            outs[(b, h)] = o[0, 0]
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    blas = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    done = len(outs)
    return {
        "value": causal_flops(1, done, n, d) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": host_cores(),
        "blas_threads": int(blas),
        "kind": "oracle",
        "sample": f"{done} of {B * H} (batch, head) pairs of the causal prefill "
                  f"[{B},{H},{n},{d}], fp64 NumPy materialised scores, {dt:.1f} s",
    }, outs


def parity_entry(got, want):
    """max-abs / mean-abs of got - want (fp64) and the bf16 output-rounding floor."""
    import numpy as np
    import torch

    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = np.abs(got - want)
    x = torch.from_numpy(np.ascontiguousarray(want))
    floor = float((x.to(torch.bfloat16).to(torch.float64) - x).abs().max())
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()), "bf16_floor": floor,
            "finite": bool(np.all(np.isfinite(got))), "elements": int(d.size)}


def parity(prefill_o, prefill_ref, pw, decode_o, lw, long_o):
    """Parity of this run's outputs against the oracle (part of the CPU-baseline leg)."""
    import numpy as np

    import oracle

    out = {"tolerance": "bf16: max-abs <= 1e-2 and mean-abs <= 1e-3 against the fp64 oracle "
                        "on the same bf16 inputs"}
    keys = sorted(prefill_ref)
    got = np.stack([prefill_o[b, h] for b, h in keys])
    want = np.stack([prefill_ref[k] for k in keys])
    out["prefill"] = dict(parity_entry(got, want), heads=len(keys))
    # the oracle's own time on each reference it computes here (algorithmic flops: 4 d per
    # admitted (query, key) pair), beside the prefill's in cpu_baseline
    t0 = time.perf_counter()
    ro, _ = oracle.decode(pw.q, pw.k_seqs, pw.v_seqs)
    dt = time.perf_counter() - t0
    H, d = pw.q.shape[1], pw.q.shape[2]
    fl = 4 * d * H * sum(int(x.shape[1]) for x in pw.k_seqs)
    out["decode"] = dict(parity_entry(decode_o, ro), oracle_s=round(dt, 3),
                         oracle_gflops=round(fl / dt / 1e9, 3))
    rows = lw["rows"].numpy()
    t0 = time.perf_counter()
    ro, _ = oracle.attention_rows(lw["q"], lw["k"], lw["v"], rows, causal=True)
    dt = time.perf_counter() - t0
    fl = 4 * lw["q"].shape[-1] * int((rows + 1).sum())
    got = np.stack([long_o[0, h, rows[h]] for h in range(rows.shape[0])])[None]
    out["long_prefill"] = dict(parity_entry(got, ro), rows=f"{rows.shape[1]} seeded rows per head",
                               oracle_s=round(dt, 3), oracle_gflops=round(fl / dt / 1e9, 3))
    return out


# --------------------------------------------------------------------------- default run
def bench_default(args, attn, workloads, torch):
    dev = torch.device("cuda:0")
    clock = ClockSampler().start()
    w3 = workloads.causal_prefill()
    lw = workloads.long_prefill()
    pw = workloads.paged_decode()
    B, H, n, d = w3["q"].shape
    q, k, v = (w3[x].to(dev) for x in "qkv")
    o = torch.empty_like(q)
    lq, lk, lv = (lw[x].to(dev) for x in "qkv")
    lo = torch.empty_like(lq)
    dq, kc, vc = pw.q.to(dev), pw.k_cache.to(dev), pw.v_cache.to(dev)
    tbl, lens = pw.block_table.to(dev), pw.seq_lens.to(dev)
    dout = torch.empty_like(dq)
    ws = torch.empty(attn.attn_decode_workspace_bytes(32, 32, 128, pw.max_seq_len),
                     dtype=torch.uint8, device=dev)
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flops3 = causal_flops(B, H, n, d)
    flops5 = causal_flops(*lq.shape)
    dbytes = decode_bytes(pw, 32, 128)

    # input copies so that a cold launch never finds its Q/K/V in the MALL (> 600 MB)
    set_bytes = 3 * q.numel() * q.element_size()
    n_sets = max(1, -(-(600 << 20) // set_bytes))
    sets = [(q, k, v)] + [(q.clone(), k.clone(), v.clone()) for _ in range(n_sets - 1)]
    launches = {"prefill": 0, "long": 0, "decode": 0}

    def prefill(i=0):
        qq, kk, vv = sets[i % n_sets]
        attn.attn_fwd(qq, kk, vv, causal=True, out=o)
        launches["prefill"] += 1

    def long_prefill():
        attn.attn_fwd(lq, lk, lv, causal=True, out=lo)
        launches["long"] += 1

    def decode():
        attn.attn_decode_paged(dq, kc, vc, tbl, lens, max_seq_len=pw.max_seq_len, out=dout,
                               workspace=ws)
        launches["decode"] += 1

    flush_val = [0]

    def flush():  # a 1 GiB write evicts the decode's cache pages from the 256 MB MALL
        flush_val[0] ^= 1
        scratch.fill_(flush_val[0])

    if args.profile_pass == "long":
        # the long prefill under sustained load: 30 launches back to back (the counters of
        # the last ones describe the settled clock)
        for _ in range(30):
            long_prefill()
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "workload": "long prefill", "launches": 30}))
        clock.stop()
        return
    if args.profile_pass:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)            # plain copy of known size: 1 GiB read + 1 GiB written
        prefill()
        decode()
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "copy_bytes": 1 << 30, "workload": "prefill"}))
        clock.stop()
        return

    clock.mark("settle")
    settle_ms, rounds = settle([prefill, decode, long_prefill], args.settle_ms / 1e3)
    clock.mark("warmup")
    for i in range(args.warmup):
        prefill(i)
        flush()
        decode()
        long_prefill()
    torch.cuda.synchronize()

    # ---- the K timed steps
    K = args.steps
    idx = {"prefill_first": launches["prefill"] + 1, "long_first": launches["long"],
           "decode_first": launches["decode"]}
    clock.mark("timed")
    e_pre, e_long = events(2), events(2)
    t0 = time.perf_counter()
    prefill(0)  # untimed: keeps the GPU busy while the event and the burst are enqueued
    e_pre[0].record()
    for _ in range(K):
        prefill(0)
    e_pre[1].record()
    dec_ms = flushed_times(decode, flush, K)
    e_long[0].record()
    for _ in range(K):
        long_prefill()
    e_long[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock.mark("stats")
    pre_avg = e_pre[0].elapsed_time(e_pre[1]) / K
    long_avg = e_long[0].elapsed_time(e_long[1]) / K
    dec_avg = sum(dec_ms) / K

    # ---- per-launch statistics and references (outside the timed steps)
    pre_stats = burst_stats(prefill, 50, 5)
    dec_stats = stats(flushed_times(decode, flush, 50),
                      "50 calls, each after a 1 GiB scratch write, between its own event pair")
    long_stats = stats(flushed_times(long_prefill, lambda: None, 50),
                       "50 launches, each between its own event pair")
    b2b_ms = burst_ms(decode, K)
    prefill(n_sets - 1)
    ce = events(2)
    ce[0].record()
    for i in range(K):
        prefill(i)
    ce[1].record()
    torch.cuda.synchronize()
    cold_ms = ce[0].elapsed_time(ce[1]) / K
    clock.mark("idle")
    clock.stop()

    tf3 = flops_rate(flops3, pre_avg)
    tf5 = flops_rate(flops5, long_avg)
    gbs = dbytes / (dec_avg * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(tf3, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded KV lengths and page permutation)",
        "config": {"workload": "causal prefill B=4 H=32 n=2048 d=128 bf16 + paged decode B=32 "
                               "H=32 d=128 lens U[1024,8192] block 16 (1 GiB scratch write "
                               "before each call) + causal prefill B=1 H=32 n=32768 d=128 bf16",
                   "batch": B, "heads": H, "kv_heads": H, "seq_len": n, "head_dim": d,
                   "causal": True, "window": 0},
        "settle": {"ms": round(settle_ms, 1), "rounds": rounds,
                   "what": "causal prefill, decode and long prefill round-robin before the "
                           "warm-up steps, for a fixed wall time"},
        "prefill": dict({"ms_avg": round(pre_avg, 5), "tflops": round(tf3, 2),
                         "frac_of_peak": round(tf3 / PEAK_BF16_TFLOPS, 4),
                         "flops": flops3, "inputs_warm": "one input set back to back (201 MB: "
                         "resident in the 256 MB MALL, as after the projection that writes it)",
                         "cold_ms_avg": round(cold_ms, 5),
                         "cold_tflops": round(flops_rate(flops3, cold_ms), 2),
                         "cold_input_sets": n_sets}, **pre_stats,
                        median_tflops=round(flops_rate(flops3, pre_stats["median_ms"]), 2)),
        "roofline": roofline_mfma(tf3, traffic=recorded_traffic("prefill")),
        "decode": dict({"value": round(gbs, 1), "unit": "GB/s", "ms_avg": round(dec_avg, 5),
                        "bytes": dbytes, "flush_bytes": FLUSH_BYTES}, **dec_stats,
                       median_gbs=round(dbytes / (dec_stats["median_ms"] * 1e-3) / 1e9, 1),
                       back_to_back={"ms_avg": round(b2b_ms, 5),
                                     "gbs": round(dbytes / (b2b_ms * 1e-3) / 1e9, 1),
                                     "note": "no scratch write between calls: part of the cache "
                                             "may be read from the MALL"},
                       roofline=roofline_hbm(gbs, recorded_traffic("decode"))),
        "long_prefill": dict({"ms_avg": round(long_avg, 5), "tflops": round(tf5, 2),
                              "flops": flops5}, **long_stats,
                             median_tflops=round(flops_rate(flops5, long_stats["median_ms"]), 2),
                             roofline=roofline_mfma(tf5)),
        "trace_index": dict(idx, note="0-based positions, in launch order, of the first timed "
                                      "launch of each kind (prefill and long told apart by "
                                      "grid size)"),
        "env": dict(env_info(), clock_timed=clock.summary({"timed"}),
                    clock_all=clock.summary({"settle", "warmup", "timed", "stats"})),
    }
    if not args.no_cpu_baseline:
        base, refs = cpu_baseline(w3["q"], w3["k"], w3["v"])
        result["cpu_baseline"] = base
        prefill(0)  # the output of the first input set (the last launch read a copy)
        torch.cuda.synchronize()
        result["parity"] = parity(o.to(torch.float64).cpu().numpy(), refs, pw,
                                  dout.to(torch.float64).cpu().numpy(), lw,
                                  lo.to(torch.float64).cpu().numpy())
    print(json.dumps(result))


# --------------------------------------------------------------------------- other legs
def bench_two_legs(args, attn, workloads, torch):
    """long | grouped | window: a prefill (and for grouped/window a decode) timed like the
    default run's legs."""
    dev = torch.device("cuda:0")
    window, kv_heads = 0, 32
    dec_cfg = ""
    if args.workload == "long":
        w = workloads.long_prefill()
        pre_cfg = "causal prefill B=1 H=32 n=32768 d=128 bf16"
    elif args.workload == "grouped":
        kv_heads = 8
        q3, k3, v3 = workloads.prefill(4, 32, 2048, 128, seed=3, kv_heads=kv_heads)
        w = dict(q=q3, k=k3, v=v3)
        pre_cfg = "causal prefill B=4 H=32 H_kv=8 n=2048 d=128 bf16"
        dec_cfg = " + paged decode B=32 H=32 H_kv=8 d=128 lens U[1024,8192] block 16"
    else:
        window = 1024
        q3, k3, v3 = workloads.prefill(1, 32, 16384, 128, seed=6)
        w = dict(q=q3, k=k3, v=v3)
        pre_cfg = "causal window-1024 prefill B=1 H=32 n=16384 d=128 bf16"
        dec_cfg = " + paged decode B=32 H=32 d=128 lens U[1024,8192] window 1024 block 16"
    B, H, n, d = w["q"].shape
    q, k, v = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    o = torch.empty_like(q)
    flops = causal_flops(B, H, n, d, window)

    def prefill():
        attn.attn_fwd(q, k, v, causal=True, window=window, out=o)

    fns = [prefill]
    dec = None
    if dec_cfg:
        if kv_heads == 32:
            pw = workloads.paged_decode()
        else:  # the decode workload's lengths, K/V drawn for kv_heads heads
            g = torch.Generator().manual_seed(4)
            dl = [int(x) for x in torch.randint(1024, 8193, (32,), generator=g)]
            pw = workloads.paged(dl, 32, 128, seed=44, max_seq_len=8192, kv_heads=kv_heads)
        dq, kc, vc = pw.q.to(dev), pw.k_cache.to(dev), pw.v_cache.to(dev)
        tbl, lens = pw.block_table.to(dev), pw.seq_lens.to(dev)
        dout = torch.empty_like(dq)
        ws = torch.empty(attn.attn_decode_workspace_bytes(32, 32, 128, pw.max_seq_len,
                                                          kv_heads=kv_heads, window=window),
                         dtype=torch.uint8, device=dev)
        dbytes = decode_bytes(pw, kv_heads, 128, window)
        scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

        def decode():
            attn.attn_decode_paged(dq, kc, vc, tbl, lens, max_seq_len=pw.max_seq_len,
                                   window=window, out=dout, workspace=ws)

        def flush():
            scratch.fill_(1)

        fns.append(decode)
        dec = (decode, flush)
        groups = []  # grouped workload: the same cache under 8 and 16 query heads per K/V head
        if args.workload == "grouped":
            gq = torch.Generator().manual_seed(45)
            for Hg in (64, 128):
                qg = torch.randn(32, Hg, 128, generator=gq).to(torch.bfloat16).to(dev)
                og = torch.empty_like(qg)
                wsg = torch.empty(attn.attn_decode_workspace_bytes(32, Hg, 128, pw.max_seq_len,
                                                                   kv_heads=kv_heads),
                                  dtype=torch.uint8, device=dev)

                def dec_g(qg=qg, og=og, wsg=wsg):
                    attn.attn_decode_paged(qg, kc, vc, tbl, lens, max_seq_len=pw.max_seq_len,
                                           out=og, workspace=wsg)

                groups.append((Hg // kv_heads, dec_g, qg.numel()))
                fns.append(dec_g)
    clock = ClockSampler().start()
    clock.mark("settle")
    settle_ms, rounds = settle(fns, args.settle_ms / 1e3)
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    clock.mark("timed")
    # launches of each kernel before the timed ones (settle rounds and warm-up steps call
    # every function once; a burst starts with one untimed launch)
    before = rounds + args.warmup
    t0 = time.perf_counter()
    pre_avg = burst_ms(prefill, args.steps)
    if dec:
        dec_ms = flushed_times(dec[0], dec[1], args.steps)
        group_ms = [(G, flushed_times(fn, dec[1], args.steps), nq) for G, fn, nq in groups]
    wall = time.perf_counter() - t0
    clock.mark("stats")
    pre_stats = burst_stats(prefill, 50, 2 if n > 8192 else 5)
    clock.mark("idle")
    clock.stop()
    tf = flops_rate(flops, pre_avg)
    result = {
        "metric": METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded KV lengths and page permutation)",
        "config": {"workload": pre_cfg + dec_cfg, "batch": B, "heads": H, "kv_heads": kv_heads,
                   "seq_len": n, "head_dim": d, "causal": True, "window": window},
        "settle": {"ms": round(settle_ms, 1)},
        "prefill": dict({"ms_avg": round(pre_avg, 5), "tflops": round(tf, 2), "flops": flops},
                        **pre_stats, clock=clock.summary({"settle", "timed", "stats"})),
        "roofline": roofline_mfma(tf),
        "trace_index": {"fwd_bf16_kernel": [before + 1, args.steps]},
    }
    if dec:
        avg = sum(dec_ms) / len(dec_ms)
        gbs = dbytes / (avg * 1e-3) / 1e9
        result["decode"] = dict({"value": round(gbs, 1), "unit": "GB/s", "ms_avg": round(avg, 5),
                                 "bytes": dbytes, "flush_bytes": FLUSH_BYTES},
                                **stats(dec_ms, f"{len(dec_ms)} calls, each after a 1 GiB "
                                                "scratch write"),
                                roofline=roofline_hbm(gbs))
        result["decode"]["heads_per_kv_head"] = 32 // kv_heads
        kern = "decode_gqa_kernel" if kv_heads < 32 else "decode_split_kernel"
        n_dec = 1 + len(group_ms)
        for i, tag in enumerate(["H32"] + [f"H{G * kv_heads}" for G, _, _ in group_ms]):
            for kname in (kern, "decode_merge_kernel"):
                result["trace_index"][f"{kname}#{tag}"] = [n_dec * before + i * args.steps,
                                                           args.steps]
        for G, ms, nq in group_ms:
            avg = sum(ms) / len(ms)
            gbytes = dbytes - 2 * pw.q.numel() * 2 + 2 * nq * 2  # the same cache, its own q, o
            gbs = gbytes / (avg * 1e-3) / 1e9
            result[f"decode_group{G}"] = dict(
                {"value": round(gbs, 1), "unit": "GB/s", "ms_avg": round(avg, 5),
                 "config": f"paged decode B=32 H={G * kv_heads} H_kv={kv_heads} d=128, the same "
                           "cache and lengths", "bytes": gbytes},
                **stats(ms, f"{len(ms)} calls, each after a 1 GiB scratch write"),
                roofline=roofline_hbm(gbs))
    print(json.dumps(result))


def bench_backward(args, attn, workloads, torch):
    dev = torch.device("cuda:0")
    w = workloads.causal_prefill()
    B, H, n, d = w["q"].shape
    g = torch.Generator().manual_seed(33)
    q, k, v = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    do = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16).to(dev)
    o, lse = attn.attn_fwd(q, k, v, causal=True, return_lse=True)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(attn.attn_bwd_workspace_bytes(B, H, n), dtype=torch.uint8, device=dev)

    def step():
        attn.attn_bwd(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)

    settle_ms, rounds = settle([step], args.settle_ms / 1e3)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = burst_ms(step, args.steps)
    wall = time.perf_counter() - t0
    st = burst_stats(step, 50, 2)
    first = rounds + args.warmup + 1
    flops = 2.5 * causal_flops(B, H, n, d)
    tf = flops_rate(flops, ms)
    print(json.dumps({
        "metric": "attn bwd TFLOPS (causal bf16, recomputation from the saved lse)",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO)",
        "config": {"workload": "causal backward B=4 H=32 n=2048 d=128 bf16 -> fp32 grads"},
        "settle": {"ms": round(settle_ms, 1)},
        "roofline": roofline_mfma(tf), "ms_avg": round(ms, 5), **st,
        "trace_index": {"bwd_dq_kernel": [first, args.steps],
                        "bwd_dkdv_kernel": [first, args.steps]}}))


def bench_fp8(args, attn, workloads, torch):
    dev = torch.device("cuda:0")
    w = workloads.causal_prefill()
    B, H, n, d = w["q"].shape
    q, k, v = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)

    def quantize():
        return (attn.attn_quantize_fp8(q), attn.attn_quantize_fp8(k),
                attn.attn_quantize_fp8(v, transpose=True))

    one = quantize()
    set_bytes = sum(x.numel() * x.element_size() for x in (one[0][0], one[1][0], one[2][0]))
    n_sets = max(1, -(-(600 << 20) // set_bytes))
    sets = [one] + [tuple((a.clone(), b.clone()) for a, b in one) for _ in range(n_sets - 1)]
    o = torch.empty(B, H, n, d, dtype=torch.bfloat16, device=dev)
    cyc = [0]

    def step(i=None):
        i = 0 if i is None else i
        (q8, sq), (k8, sk), (v8, sv) = sets[i % n_sets]
        attn.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=True, out=o)

    def cold():
        cyc[0] += 1
        step(cyc[0])

    settle_ms, rounds = settle([step, quantize], args.settle_ms / 1e3)
    for _ in range(args.warmup):
        quantize()
        step()
    torch.cuda.synchronize()
    q_ms = burst_ms(quantize, args.steps)
    t0 = time.perf_counter()
    ms = burst_ms(step, args.steps)
    wall = time.perf_counter() - t0
    st = burst_stats(step, 50, 5)
    cold_ms = burst_ms(cold, args.steps)
    flops = causal_flops(B, H, n, d)
    tf = flops_rate(flops, ms)
    print(json.dumps({
        "metric": "attn fwd TFLOPS (causal prefill, FP8 E4M3 operands, per-block scales)",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3",
        "data": "synthetic (seeded N(0,1) Q/K/V, bf16 then block-quantised)",
        "config": {"workload": "causal prefill B=4 H=32 n=2048 d=128, E4M3 operands, bf16 output"},
        "settle": {"ms": round(settle_ms, 1)},
        "roofline": roofline_mfma(tf, PEAK_FP8_TFLOPS),
        "ms_avg": round(ms, 5), **st, "cold_ms_avg": round(cold_ms, 5),
        "cold_tflops": round(flops_rate(flops, cold_ms), 2), "cold_input_sets": n_sets,
        "quantize_ms_avg": round(q_ms, 5),
        "trace_index": {"fwd_fp8_kernel": [rounds + args.warmup + 1, args.steps]}}))


def bench_cp(args, attn, workloads, torch):
    """One device's share of sequence-parallel causal attention over the long-context workload.

    [1, 32, 32768, 128] cut into 2G = 16 chunks of 2048 tokens for G = 8 devices, device g
    owning query chunks g and 2G-1-g (zig-zag: every device gets 17 chunk pairs of causal
    work).  `--workload cp`: the K/V shards gathered first (an all-gather over the node's
    direct links), the share is one attn_fwd_chunk per owned query chunk against the whole
    K/V (the causal mask stops it at the chunk's last position).  `--workload cp-ring`: the
    form that consumes K/V chunks one at a time as a ring delivers them: attn_fwd of the
    query chunk against each K/V chunk (causal on the diagonal one) and one attn_merge of
    the c+1 results.  All data is resident on this one GPU: the exchange itself is not timed.
    """
    dev = torch.device("cuda:0")
    w = workloads.long_prefill()
    q, k, v = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    B, H, n, d = q.shape
    G, g_dev = 8, 0
    C = 2 * G
    c = n // C
    chunk = lambda t, j: t[:, :, j * c:(j + 1) * c].contiguous()
    owned = [g_dev, C - 1 - g_dev]
    ring = args.workload == "cp-ring"
    Qc = {i: chunk(q, i) for i in owned}
    outs = {i: torch.empty(B, H, c, d, dtype=torch.bfloat16, device=dev) for i in owned}
    out_lse = {i: torch.empty(B, H, c, dtype=torch.float32, device=dev) for i in owned}
    if ring:
        Kc = [chunk(k, j) for j in range(max(owned) + 1)]
        Vc = [chunk(v, j) for j in range(max(owned) + 1)]
        del k, v
        parts = {i: torch.empty(i + 1, B, H, c, d, dtype=torch.bfloat16, device=dev) for i in owned}
        lses = {i: torch.empty(i + 1, B, H, c, dtype=torch.float32, device=dev) for i in owned}
    del q

    def step():
        for i in owned:
            if ring:
                for j in range(i + 1):
                    attn.attn_fwd(Qc[i], Kc[j], Vc[j], causal=(j == i), out=parts[i][j],
                                  lse=lses[i][j])
                attn.attn_merge(parts[i], lses[i], out=outs[i], lse=out_lse[i])
            else:
                attn.attn_fwd_chunk(Qc[i], k, v, i * c, causal=True, out=outs[i], lse=out_lse[i])

    settle_ms, rounds = settle([step], args.settle_ms / 1e3)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = burst_ms(step, args.steps)
    wall = time.perf_counter() - t0
    per_step = sum(i + 1 for i in owned) if ring else len(owned)  # forward launches per step
    index = {"fwd_bf16_kernel": [(rounds + args.warmup + 1) * per_step, args.steps * per_step]}
    if ring:
        index["merge_kernel"] = [(rounds + args.warmup + 1) * len(owned), args.steps * len(owned)]
    full = 4.0 * d * B * H * c * c                  # an unmasked chunk pair
    diag = 4.0 * d * B * H * c * (c + 1) / 2        # a causal diagonal chunk
    n_full = sum(owned)
    flops = n_full * full + len(owned) * diag
    tf = flops_rate(flops, ms)
    form = (f"{n_full} unmasked + {len(owned)} causal chunk pairs + {len(owned)} merges, K/V "
            f"chunks as a ring delivers them" if ring else
            f"one chunk launch per owned query chunk against the gathered K/V")
    print(json.dumps({
        "metric": "sequence-parallel causal attention: one device's share, TFLOPS",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V of the long-context workload)",
        "config": {"workload": f"causal prefill B=1 H=32 n=32768 d=128 in {C} chunks of {c} for "
                               f"{G} devices (zig-zag); device {g_dev}: query chunks {owned}; "
                               f"{form}; the K/V exchange itself not included"},
        "settle": {"ms": round(settle_ms, 1)},
        "roofline": roofline_mfma(tf), "ms_avg": round(ms, 5), "trace_index": index}))


def bench_shapes(args, attn, workloads, torch):
    """Throughput across shapes: per shape, 0.5 s of launches to settle, then at least 0.2 s
    of back-to-back launches between one event pair.  Inputs are seeded N(0,1) tensors made
    on the device; decode puts every sequence at the stated length, its pages in a random
    permutation of the pool, and writes 1 GiB of scratch before each timed call."""
    dev = "cuda"

    def timed(fn, reps=10):
        settle([fn], 0.5)
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        per = time.perf_counter() - t0
        return burst_ms(fn, max(reps, int(0.2 / max(per, 1e-6))))

    def emit(kind, shape, ms, rate, unit, peak):
        print(json.dumps({"shape_kind": kind, "shape": shape, "ms": round(ms, 5),
                          "rate": round(rate, 2), "unit": unit, "frac": round(rate / peak, 4)}),
              flush=True)

    def qkv(B, H, Hkv, n, d=128, dtype=torch.bfloat16):
        g = torch.Generator(device=dev).manual_seed(1)
        mk = lambda h: torch.randn(B, h, n, d, generator=g, device=dev).to(dtype)
        return mk(H), mk(Hkv), mk(Hkv)

    for (B, H, Hkv, n, d, causal) in [(32, 32, 32, 512, 128, True), (16, 32, 32, 1024, 128, True),
                                      (4, 32, 32, 2048, 128, True), (4, 32, 32, 2048, 128, False),
                                      (1, 32, 32, 4096, 128, True), (4, 32, 32, 4096, 128, False),
                                      (2, 32, 32, 8192, 128, True), (1, 32, 32, 16384, 128, True),
                                      (1, 32, 32, 32768, 128, True), (4, 32, 8, 2048, 128, True),
                                      (1, 64, 8, 8192, 128, True), (4, 32, 32, 2048, 64, True),
                                      (1, 32, 32, 16384, 64, True)]:
        q, k, v = qkv(B, H, Hkv, n, d)
        o = torch.empty_like(q)
        ms = timed(lambda: attn.attn_fwd(q, k, v, causal=causal, out=o))
        pairs = n * (n + 1) / 2 if causal else n * n
        emit("prefill bf16", f"[{B},{H},{n},{d}] kv_heads {Hkv} {'causal' if causal else 'full'}",
             ms, 4 * d * B * H * pairs / ms / 1e9, "TFLOP/s", PEAK_BF16_TFLOPS)
        del q, k, v, o
    for (B, H, n, d, causal, lens) in [(1, 1, 256, 64, False, None),
                                       (4, 4, 1000, 64, True, [1000, 900, 500, 17]),
                                       (4, 32, 2048, 128, True, None)]:
        q, k, v = qkv(B, H, H, n, d, torch.float32)
        o = torch.empty_like(q)
        ms = timed(lambda: attn.attn_fwd(q, k, v, causal=causal, seq_lens=lens, out=o))
        pairs = (B * (n * (n + 1) / 2 if causal else n * n) if lens is None else
                 sum(L * (L + 1) / 2 if causal else L * L for L in lens))
        emit("prefill fp32 (fp64 scores)", f"[{B},{H},{n},{d}] {'causal' if causal else 'full'}"
             + (f" lens {lens}" if lens else ""), ms, 4 * d * H * pairs / ms / 1e9, "TFLOP/s",
             PEAK_FP64_TFLOPS)
        del q, k, v, o
    for (B, H, n, causal) in [(4, 32, 2048, True), (1, 32, 8192, True), (4, 32, 4096, False)]:
        q, k, v = qkv(B, H, H, n)
        q8, k8, v8 = (attn.attn_quantize_fp8(q), attn.attn_quantize_fp8(k),
                      attn.attn_quantize_fp8(v, transpose=True))
        o = torch.empty_like(q)
        ms = timed(lambda: attn.attn_fwd_fp8(q8[0], k8[0], v8[0], q8[1], k8[1], v8[1],
                                             causal=causal, out=o))
        pairs = n * (n + 1) / 2 if causal else n * n
        emit("prefill fp8", f"[{B},{H},{n},128] {'causal' if causal else 'full'}", ms,
             4 * 128 * B * H * pairs / ms / 1e9, "TFLOP/s", PEAK_FP8_TFLOPS)
        del q, k, v, o, q8, k8, v8
    for (B, H, Hkv, n, causal) in [(4, 32, 32, 2048, True), (4, 32, 32, 2048, False),
                                   (1, 32, 32, 8192, True), (4, 32, 8, 2048, True)]:
        q, k, v = qkv(B, H, Hkv, n)
        do = torch.randn_like(q)
        o, lse = attn.attn_fwd(q, k, v, causal=causal, return_lse=True)
        grads = attn.attn_bwd(q, k, v, o, do, lse, causal=causal)
        ws = torch.empty(attn.attn_bwd_workspace_bytes(B, H, n), dtype=torch.uint8, device=dev)
        ms = timed(lambda: attn.attn_bwd(q, k, v, o, do, lse, causal=causal, dq=grads[0],
                                         dk=grads[1], dv=grads[2], workspace=ws))
        pairs = n * (n + 1) / 2 if causal else n * n
        emit("backward", f"[{B},{H},{n},128] kv_heads {Hkv} {'causal' if causal else 'full'}",
             ms, 2.5 * 4 * 128 * B * H * pairs / ms / 1e9, "TFLOP/s", PEAK_BF16_TFLOPS)
        del q, k, v, do, o, lse, grads, ws
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    for (B, H, Hkv, L, window) in [(8, 32, 32, 32768, 0), (64, 32, 32, 4096, 0),
                                   (256, 32, 32, 1024, 0), (64, 32, 8, 4096, 0),
                                   (64, 64, 8, 8192, 0), (64, 128, 8, 4096, 0),
                                   (64, 32, 32, 8192, 1024)]:
        nbps = L // 16
        nb = B * nbps
        g = torch.Generator(device=dev).manual_seed(2)
        kc = torch.randn(nb, Hkv, 16, 128, generator=g, device=dev).to(torch.bfloat16)
        vc = torch.randn(nb, Hkv, 16, 128, generator=g, device=dev).to(torch.bfloat16)
        bt = torch.randperm(nb, generator=g, device=dev).to(torch.int32).view(B, nbps).contiguous()
        q = torch.randn(B, H, 128, generator=g, device=dev).to(torch.bfloat16)
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        ws = torch.empty(attn.attn_decode_workspace_bytes(B, H, 128, L, 0, kv_heads=Hkv,
                                                          window=window),
                         dtype=torch.uint8, device=dev)
        fn = lambda: attn.attn_decode_paged(q, kc, vc, bt, lens, max_seq_len=L, window=window,
                                            out=out, workspace=ws)
        settle([fn], 0.3)
        ms = statistics.median(flushed_times(fn, lambda: scratch.fill_(1), 30))
        keys = min(L, window) if window else L
        nbytes = B * Hkv * keys * 128 * 2 * 2
        emit("decode (flushed, median of 30)", f"B={B} H={H} kv_heads {Hkv} len {L}"
             + (f" window {window}" if window else ""), ms, nbytes / ms / 1e6, "GB/s",
             PEAK_HBM_GBS)
        del kc, vc, bt, q, out, ws


# --------------------------------------------------------------------------- profiles
def bench_ceilings(args, attn, workloads, torch):
    """The device's own ceilings, measured by the probe kernels of the library
    (include/attn_probe.h), each settled for about a second and then timed in 10 bursts of
    3 back-to-back launches (median): dense matrix-core rate in bf16 and fp8 (blocks of
    ones times blocks of twos, two accumulation chains per wave, two workgroups per CU),
    v_exp_f32 rate (eight chains x <- 2^(-x) per lane), and HBM reads of a 2 GiB buffer,
    streamed and as 4 KiB pages in a seeded random order (the paged decode's access), the
    latter also after a 1 GiB write per call (the flushed decode's condition).
    Every probe's checksum is verified against the value the work must produce."""
    from online_softmax_attn_amd import binding as b

    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    clock = ClockSampler().start()
    checks = {}
    line = {}

    def timed(name, fn, work, unit_scale):
        clock.mark(name)
        settle([fn], 1.0)
        ms = [burst_ms(fn, 3) for _ in range(10)]
        med = statistics.median(ms)
        clock.mark("idle")
        rate = work / (med * 1e-3) / unit_scale
        return rate, stats(ms, "10 bursts of 3 back-to-back launches (burst time / 3)")

    # matrix cores: per wave `iters` rounds of 4 products; flops per product 2*32*32*k
    blocks = 16 * cus
    mf = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    for key, fp8, iters, k, peak in (("mfma_bf16", 0, 8192, 16, PEAK_BF16_TFLOPS),
                                     ("mfma_fp8", 1, 4096, 64, PEAK_FP8_TFLOPS)):
        flops = blocks * 4 * iters * 2 * 2 * 32 * 32 * k
        fn = (lambda fp8=fp8, iters=iters: b.attn_probe_mfma(fp8, blocks, iters, out=mf))
        tf, st = timed(key, fn, flops, 1e12)
        torch.cuda.synchronize()
        checks[key] = bool(torch.all(mf == float(64 * k * iters)).item())
        line[key] = {"tflops": round(tf, 1), "peak": peak, "frac": round(tf / peak, 4),
                     "flops_per_launch": flops, **st,
                     "clock": clock.summary({key})}

    # transcendental rate
    eb, iters = 16 * cus, 4096
    eo = torch.empty(eb * b.ATTN_PROBE_THREADS, dtype=torch.float32, device=dev)
    exps = eb * b.ATTN_PROBE_THREADS * iters * 8
    rate, st = timed("exp", lambda: b.attn_probe_exp(eb, iters, out=eo), exps, 1e9)
    torch.cuda.synchronize()
    fixed = 0.641185744504986  # x = 2^(-x)
    checks["exp"] = bool(torch.all((eo - 8 * fixed).abs() < 1e-4).item())
    line["exp"] = {"gexp_per_s": round(rate, 1), "exps_per_launch": exps, **st,
                   "clock": clock.summary({"exp"})}

    # HBM reads: 2 GiB of seeded words, streamed and as pages in a seeded random order
    nbytes = 2 << 30
    g = torch.Generator(device=dev)
    g.manual_seed(20260924)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev,
                        generator=g)
    want = int(sum(int(c.to(torch.int64).sum().item()) for c in src.split(1 << 26))) % 2**32
    rb = 8 * cus
    ro = torch.empty(rb * b.ATTN_PROBE_THREADS, dtype=torch.int32, device=dev)
    gbs, st = timed("hbm_stream", lambda: b.attn_probe_read(src, rb, out=ro), nbytes, 1e9)
    torch.cuda.synchronize()
    checks["hbm_stream"] = int(ro.to(torch.int64).sum().item()) % 2**32 == want
    line["hbm_stream"] = {"gbs": round(gbs, 1), "peak": PEAK_HBM_GBS,
                          "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes, **st}
    pages = nbytes // 4096
    gp = torch.Generator().manual_seed(4)
    order = torch.randperm(pages, generator=gp).to(torch.int32).to(dev)
    gbs, st = timed("hbm_pages_4k", lambda: b.attn_probe_read_pages(src, order, rb, out=ro),
                    nbytes, 1e9)
    torch.cuda.synchronize()
    checks["hbm_pages_4k"] = int(ro.to(torch.int64).sum().item()) % 2**32 == want
    line["hbm_pages_4k"] = {"gbs": round(gbs, 1), "peak": PEAK_HBM_GBS,
                            "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
                            "pages": pages, **st}
    # the same read after a 1 GiB write, as the flushed decode runs: the caches then hold
    # dirty lines that the reads must evict first
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush_val = [0]

    def flush():
        flush_val[0] ^= 1
        scratch.fill_(flush_val[0])

    ms = flushed_times(lambda: b.attn_probe_read_pages(src, order, rb, out=ro), flush, 20)
    torch.cuda.synchronize()
    checks["hbm_pages_4k_flushed"] = int(ro.to(torch.int64).sum().item()) % 2**32 == want
    med = statistics.median(ms)
    line["hbm_pages_4k_flushed"] = {
        "gbs": round(nbytes / (med * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
        "frac": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bytes": nbytes,
        **stats(ms, "20 calls, each after a 1 GiB scratch write (median)")}
    del scratch
    clock.stop()

    bf = line["mfma_bf16"]
    out = {"metric": "machine ceilings (probe kernels of libattn.so): dense bf16 MFMA TFLOP/s",
           "value": bf["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": 10,
           "warmup": 0, "ms_per_step": bf["median_ms"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (blocks of ones and twos; seeded random words for the reads)",
           "config": {"workload": "ceilings: matrix-core, exp and HBM-read probes",
                      "compute_units": cus},
           "roofline": roofline_mfma(bf["tflops"]), **line, "checksums": checks,
           "env": env_info()}
    print(json.dumps(out), flush=True)
    if not all(checks.values()):
        print(f"probe checksum mismatch: {checks}", file=sys.stderr)
        sys.exit(1)


def record_traffic(fetch_csv, write_csv):
    """profiles/traffic.json from FETCH_SIZE / WRITE_SIZE runs of --profile-pass."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = ("copy" if "copyBuffer" in name else "prefill" if "fwd_bf16_kernel" in name
                   else "decode_split" if "decode_split_kernel" in name
                   else "decode_merge" if "decode_merge_kernel" in name else None)
            if key:
                vals.setdefault(key, []).append(float(row["Counter_Value"]) * 1024.0)  # KiB -> B
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    f_scale = copy_bytes / max(fetch["copy"])   # the 1 GiB copy reads 1 GiB
    w_scale = copy_bytes / max(write["copy"])   # and writes 1 GiB
    out = {"scale": {"FETCH_SIZE": round(f_scale, 4), "WRITE_SIZE": round(w_scale, 4)},
           "source": "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE -- python bench.py --profile-pass"}
    out["prefill"] = {"kernel_hash": kernel_hash(KERNEL_FILES["prefill"]),
                      "fetch_bytes": fetch["prefill"][0] * f_scale,
                      "write_bytes": write["prefill"][0] * w_scale}
    out["prefill"]["bytes_per_launch"] = out["prefill"]["fetch_bytes"] + out["prefill"]["write_bytes"]
    dec = {k: fetch[k][0] * f_scale + write[k][0] * w_scale for k in ("decode_split", "decode_merge")}
    out["decode"] = {"kernel_hash": kernel_hash(KERNEL_FILES["decode"]),
                     "split_bytes": dec["decode_split"], "merge_bytes": dec["decode_merge"],
                     "bytes_per_launch": dec["decode_split"] + dec["decode_merge"]}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def summarize_trace_legs(rows, ti):
    """Summary for the other legs: `trace_index` maps "kernel[#tag]" to [first, count], the
    timed launches among those whose name contains `kernel`, in launch order."""
    out = ["| kernel (timed launches) | launches in the run | timed | avg (us) | median (us) | "
           "min (us) | max (us) |", "|---|---|---|---|---|---|---|"]
    for key, (first, count) in ti.items():
        kname = key.split("#")[0]
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
             if kname in r["Kernel_Name"]]
        timed = d[first:first + count]
        if not timed:
            out.append(f"| {key} | {len(d)} | 0 | | | | |")
            continue
        out.append(f"| {key} | {len(d)} | {len(timed)} | {sum(timed) / len(timed):.2f} | "
                   f"{statistics.median(timed):.2f} | {min(timed):.2f} | {max(timed):.2f} |")
    print("\n".join(out))


def summarize_trace(trace_csv, line_file):
    """Markdown summary of a rocprofv3 kernel trace of a default run, checked against the
    run's JSON line: the average duration over exactly the timed launches of each leg."""
    import csv

    line = None
    for raw in open(line_file):
        raw = raw.strip()
        if raw.startswith("{") and '"metric"' in raw:
            line = json.loads(raw)
    if line is None:
        raise SystemExit(f"{line_file}: no bench JSON line")
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by_kind = {}
    names = {}
    for r in rows:
        name = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
        if r.get("Grid_Size"):
            grid = int(r["Grid_Size"])
        else:
            grid = 1
            for ax in "XYZ":
                grid *= int(r.get(f"Grid_Size_{ax}") or 1)
        if "fwd_bf16_kernel" in name:
            kind = "long" if grid >= 256 * 8192 else "prefill"
        elif "decode_split_kernel" in name or "decode_gqa_kernel" in name:
            kind = "decode_split"
        elif "decode_merge_kernel" in name:
            kind = "decode_merge"
        else:
            kind = "other"
        short = re.search(r"\w+_kernel(<[^>]*>)?", name)
        names.setdefault(kind, set()).add(short.group(0) if short else name[:80])
        by_kind.setdefault(kind, []).append(dur)
    K = int(line["steps"])
    ti = line["trace_index"]
    if all(isinstance(x, list) for x in ti.values()):
        return summarize_trace_legs(rows, ti)
    out = ["| kernel | launches | avg over all (us) | avg over the timed launches (us) | line (us) |",
           "|---|---|---|---|---|"]

    def row(kind, first, line_us):
        d = by_kind.get(kind, [])
        timed = d[first:first + K]
        avg_t = sum(timed) / len(timed) if timed else float("nan")
        out.append(f"| {kind}: {', '.join(sorted(names.get(kind, [])))} | {len(d)} | "
                   f"{sum(d) / max(len(d), 1):.2f} | {avg_t:.2f} | "
                   f"{'' if line_us is None else f'{line_us:.2f}'} |")
        return avg_t

    pre = row("prefill", ti["prefill_first"], line["prefill"]["ms_avg"] * 1e3)
    lng = row("long", ti["long_first"], line["long_prefill"]["ms_avg"] * 1e3)
    spl = row("decode_split", ti["decode_first"], None)
    mrg = row("decode_merge", ti["decode_first"], None)
    out.append(f"| decode split + merge | | | {spl + mrg:.2f} | "
               f"{line['decode']['ms_avg'] * 1e3:.2f} (event pair around the call) |")
    out.append("")
    out.append(f"Timed causal prefill: trace {pre:.2f} us vs line {line['prefill']['ms_avg'] * 1e3:.2f} us "
               f"({(line['prefill']['ms_avg'] * 1e3 / pre - 1) * 100:+.2f}%); long prefill: trace "
               f"{lng:.2f} us vs line {line['long_prefill']['ms_avg'] * 1e3:.2f} us "
               f"({(line['long_prefill']['ms_avg'] * 1e3 / lng - 1) * 100:+.2f}%).")
    print("\n".join(out))


def main():
    if len(sys.argv) == 4 and sys.argv[1] == "--record-traffic":
        record_traffic(sys.argv[2], sys.argv[3])
        return
    if len(sys.argv) == 4 and sys.argv[1] == "--summarize-trace":
        summarize_trace(sys.argv[2], sys.argv[3])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    # the shader clock ramps up over tens of ms of sustained work: the legs run for this long
    # before the warm-up steps, whatever --warmup is
    ap.add_argument("--settle-ms", type=float, default=400.0)
    ap.add_argument("--workload", choices=["prefill", "long", "backward", "grouped", "window",
                                           "fp8", "cp", "cp-ring", "shapes", "ceilings"],
                    default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-pass", nargs="?", const="prefill", choices=["prefill", "long"],
                    default=None)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU sharding is a design, not a build", file=sys.stderr)
        sys.exit(2)

    import torch

    import online_softmax_attn_amd as attn
    import workloads

    torch.cuda.set_device(torch.device("cuda:0"))
    attn.lib()
    legs = {"prefill": bench_default, "long": bench_two_legs, "grouped": bench_two_legs,
            "window": bench_two_legs, "backward": bench_backward, "fp8": bench_fp8,
            "cp": bench_cp, "cp-ring": bench_cp, "shapes": bench_shapes,
            "ceilings": bench_ceilings}
    legs[args.workload](args, attn, workloads, torch)


if __name__ == "__main__":
    main()
