"""attn_decode_paged_noalloc (the decode entry point that allocates nothing) through the C
ABI: two calls in a row, the second on a smaller input, each against attn_decode_paged with a
caller workspace (same kernels, same split: identical bytes) and against the oracle within
the bf16 bounds; a request past the fixed scratch array is refused before anything runs."""

import numpy as np
import pytest
import torch

import online_softmax_attn_amd as attn
import oracle
import workloads
from metrics import errs, to64

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 1e-2, 1e-3


def _device_inputs(w):
    return (w.q.cuda(), w.k_cache.cuda(), w.v_cache.cuda(), w.block_table.cuda(),
            w.seq_lens.cuda())


@pytest.mark.parametrize("H,Hkv", [(32, 32), (32, 4)])
def test_noalloc_decode_matches_the_workspace_entry_point_twice(H, Hkv):
    cases = [([8000, 1024, 5000, 7777] * 4, 4096), ([300, 17, 1], 0)]   # second call smaller
    for lens, window in cases:
        w = workloads.paged(lens, H, 128, seed=len(lens) + H + Hkv, kv_heads=Hkv,
                            max_seq_len=max(lens), poison=True)
        q, kc, vc, tbl, sl = _device_inputs(w)
        print(f"case: noalloc decode B={len(lens)} H={H} Hkv={Hkv} window={window}", flush=True)
        need = attn.attn_decode_workspace_bytes(len(lens), H, 128, w.max_seq_len, kv_heads=Hkv,
                                                window=window)
        assert 0 < need <= attn.ATTN_NOALLOC_SCRATCH_BYTES
        ref = torch.full_like(q, float("nan"))
        ref_lse = torch.full(q.shape[:2], float("nan"), device="cuda")
        attn.attn_decode_paged(q, kc, vc, tbl, sl, max_seq_len=w.max_seq_len, window=window,
                               out=ref, lse=ref_lse)
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:2], float("nan"), device="cuda")
        attn.attn_decode_paged_noalloc(q, kc, vc, tbl, sl, max_seq_len=w.max_seq_len,
                                       window=window, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
        ro, _ = oracle.decode(w.q, w.k_seqs, w.v_seqs, window=window)
        mx, mean = errs(to64(out), ro)
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)


def test_noalloc_decode_refuses_partials_past_the_scratch_array():
    B, H = 64, 64
    w = workloads.paged([16] * B, H, 128, seed=9, max_seq_len=65536)
    q, kc, vc, tbl, sl = _device_inputs(w)
    need = attn.attn_decode_workspace_bytes(B, H, 128, 65536)
    assert need > attn.ATTN_NOALLOC_SCRATCH_BYTES
    out = torch.zeros_like(q)
    with pytest.raises(attn.AttnError) as e:
        attn.attn_decode_paged_noalloc(q, kc, vc, tbl, sl, max_seq_len=65536, out=out)
    assert e.value.status == attn.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 0).all())     # nothing ran
