"""Throughput of the library across shapes, under sustained load (one MI355X).

For each shape: at least 0.5 s of launches to warm up (the shader clock settles), then at
least 0.2 s of back-to-back launches timed with HIP events on the current stream.  Inputs are
seeded N(0,1) tensors made on the device; decode puts every sequence at the stated length,
its pages in a random permutation of the pool.  FLOP/s count admitted (query, key) pairs,
4 * head_dim flops each (the backward 2.5 times that); decode counts the K/V bytes of the
admitted tokens.  Prints markdown table rows.  `python bench.py` is the headline measurement;
this script only widens it to more shapes.
"""
import time

import torch

import online_softmax_attn_amd as attn

dev = 'cuda'
PEAK, PEAK8, HBM = 2516.6, 5000.0, 8000.0  # MI355X dense bf16, dense fp8 (TFLOP/s), HBM (GB/s)

def timed(fn, reps=10):
    t0 = time.time(); k = 0
    while time.time() - t0 < 0.5 or k < 5:
        fn(); k += 1
        if k % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per = (time.time() - t0) / k
    reps = max(reps, int(0.2 / max(per, 1e-6)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record(); torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps

def qkv(B, H, Hkv, n):
    g = torch.Generator(device=dev).manual_seed(1)
    mk = lambda h: torch.randn(B, h, n, 128, generator=g, device=dev).to(torch.bfloat16)
    return mk(H), mk(Hkv), mk(Hkv)

print("== prefill bf16", flush=True)
for (B, H, Hkv, n, causal) in [(32, 32, 32, 512, True), (16, 32, 32, 1024, True), (4, 32, 32, 2048, True),
                               (4, 32, 32, 2048, False), (1, 32, 32, 4096, True), (4, 32, 32, 4096, False),
                               (2, 32, 32, 8192, True), (1, 32, 32, 16384, True), (1, 32, 32, 32768, True),
                               (4, 32, 8, 2048, True), (1, 64, 8, 8192, True)]:
    q, k, v = qkv(B, H, Hkv, n)
    o = torch.empty_like(q)
    ms = timed(lambda: attn.attn_fwd(q, k, v, causal=causal, out=o))
    pairs = n * (n + 1) / 2 if causal else n * n
    tf = 4 * 128 * B * H * pairs / ms / 1e9
    print(f"| [{B},{H},{n},128] kv_heads {Hkv} {'causal' if causal else 'full'} | {ms*1e3:.1f} µs | {tf:.1f} | {tf/PEAK*100:.1f}% |", flush=True)
    del q, k, v, o

print("== fp32 (fp64 scores)", flush=True)
for (B, H, n, d, causal, lens) in [(1, 1, 256, 64, False, None), (4, 4, 1000, 64, True, [1000, 900, 500, 17]),
                                   (4, 32, 2048, 128, True, None)]:
    gf = torch.Generator(device=dev).manual_seed(1)
    q, k, v = (torch.randn(B, H, n, d, generator=gf, device=dev) for _ in range(3))
    o = torch.empty_like(q)
    ms = timed(lambda: attn.attn_fwd(q, k, v, causal=causal, seq_lens=lens, out=o))
    if lens is None:
        pairs = B * (n * (n + 1) / 2 if causal else n * n)
    else:
        pairs = sum(L * (L + 1) / 2 if causal else L * L for L in lens)
    tf = 4 * d * H * pairs / ms / 1e9
    print(f"| fp32 [{B},{H},{n},{d}] {'causal' if causal else 'full'}{' lens ' + str(lens) if lens else ''} | {ms*1e3:.1f} µs | {tf:.2f} | {tf/78.6*100:.1f}% of fp64 |", flush=True)
    del q, k, v, o

print("== fp8", flush=True)
for (B, H, n, causal) in [(4, 32, 2048, True), (1, 32, 8192, True), (4, 32, 4096, False)]:
    q, k, v = qkv(B, H, H, n)
    q8, k8, v8 = attn.attn_quantize_fp8(q), attn.attn_quantize_fp8(k), attn.attn_quantize_fp8(v, transpose=True)
    o = torch.empty_like(q)
    ms = timed(lambda: attn.attn_fwd_fp8(q8[0], k8[0], v8[0], q8[1], k8[1], v8[1], causal=causal, out=o))
    pairs = n * (n + 1) / 2 if causal else n * n
    tf = 4 * 128 * B * H * pairs / ms / 1e9
    print(f"| fp8 [{B},{H},{n},128] {'causal' if causal else 'full'} | {ms*1e3:.1f} µs | {tf:.1f} | {tf/PEAK8*100:.1f}% |", flush=True)
    del q, k, v, o, q8, k8, v8

print("== backward", flush=True)
for (B, H, Hkv, n, causal) in [(4, 32, 32, 2048, True), (4, 32, 32, 2048, False), (1, 32, 32, 8192, True), (4, 32, 8, 2048, True)]:
    q, k, v = qkv(B, H, Hkv, n)
    do = torch.randn_like(q)
    o, lse = attn.attn_fwd(q, k, v, causal=causal, return_lse=True)
    grads = attn.attn_bwd(q, k, v, o, do, lse, causal=causal)
    ws = torch.empty(attn.attn_bwd_workspace_bytes(B, H, n), dtype=torch.uint8, device=dev)
    ms = timed(lambda: attn.attn_bwd(q, k, v, o, do, lse, causal=causal, dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws))
    pairs = n * (n + 1) / 2 if causal else n * n
    tf = 2.5 * 4 * 128 * B * H * pairs / ms / 1e9
    print(f"| bwd [{B},{H},{n},128] kv_heads {Hkv} {'causal' if causal else 'full'} | {ms*1e3:.1f} µs | {tf:.1f} | {tf/PEAK*100:.1f}% |", flush=True)
    del q, k, v, do, o, lse, grads, ws

print("== decode", flush=True)
for (B, H, Hkv, L, window) in [(8, 32, 32, 32768, 0), (64, 32, 32, 4096, 0), (256, 32, 32, 1024, 0),
                               (64, 32, 8, 4096, 0), (64, 64, 8, 8192, 0), (64, 32, 32, 8192, 1024)]:
    nbps = L // 16
    nb = B * nbps
    g = torch.Generator(device=dev).manual_seed(2)
    kc = torch.randn(nb, Hkv, 16, 128, generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn(nb, Hkv, 16, 128, generator=g, device=dev).to(torch.bfloat16)
    bt = torch.randperm(nb, generator=g, device=dev).to(torch.int32).view(B, nbps).contiguous()
    q = torch.randn(B, H, 128, generator=g, device=dev).to(torch.bfloat16)
    lens = [L] * B
    out = torch.empty_like(q)
    ws = torch.empty(attn.attn_decode_workspace_bytes(B, H, 128, L, 0, kv_heads=Hkv, window=window), dtype=torch.uint8, device=dev)
    ms = timed(lambda: attn.attn_decode_paged(q, kc, vc, bt, lens, max_seq_len=L, window=window, out=out, workspace=ws), reps=20)
    keys = min(L, window) if window else L
    nbytes = B * Hkv * keys * 128 * 2 * 2
    gbs = nbytes / ms / 1e6
    print(f"| decode B={B} H={H} kv_heads {Hkv} len {L}{' window %d' % window if window else ''} | {ms*1e3:.1f} µs | {gbs:.0f} GB/s | {gbs/HBM*100:.1f}% |", flush=True)
    del kc, vc, bt, q, out, ws
