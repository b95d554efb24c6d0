"""Exact scaled dot-product attention for MI355X (gfx950): Python face of libattn.so.

Entry points mirror the C ABI in include/attn.h:
    attn_fwd                      prefill over [B, H, n, d] (fp32 or bf16), causal/length masks
    attn_fwd_chunk                a chunk of queries at an offset into a longer key sequence
    attn_bwd                      gradients dq, dk, dv by recomputation from the saved lse
    attn_bwd_workspace_bytes      workspace size the backward pass needs
    attn_decode_paged             one query per sequence against a paged bf16 K/V cache
    attn_decode_workspace_bytes   workspace size the decode needs
    attn_decode_paged_noalloc     the decode without a workspace (allocates nothing)
    attn_quantize_fp8             bf16 -> FP8 E4M3 codes with one scale per 64-row block
    attn_fwd_fp8                  prefill on E4M3 operands (bf16 output)
    attn_merge                    join results over disjoint key sets by their lse
    attn_status_str, attn_abi_version

Measurement kernels (include/attn_probe.h: matrix-core, exp and HBM-read rates of the
device) are in `binding` under their C names (attn_probe_mfma, attn_probe_exp,
attn_probe_read, attn_probe_read_pages); `python bench.py --workload ceilings` runs them.
"""

from .binding import (
    ATTN_BF16,
    ATTN_ERR_INVALID,
    ATTN_ERR_LAUNCH,
    ATTN_ERR_UNSUPPORTED,
    ATTN_ERR_WORKSPACE,
    ATTN_F32,
    ATTN_NOALLOC_SCRATCH_BYTES,
    ATTN_OK,
    LIB_PATH,
    AttnError,
    attn_abi_version,
    attn_bwd,
    attn_bwd_workspace_bytes,
    attn_decode_paged,
    attn_decode_paged_noalloc,
    attn_decode_workspace_bytes,
    attn_fwd,
    attn_fwd_chunk,
    attn_fwd_fp8,
    attn_merge,
    attn_quantize_fp8,
    attn_status_str,
    lib,
)

__all__ = [
    "ATTN_BF16",
    "ATTN_ERR_INVALID",
    "ATTN_ERR_LAUNCH",
    "ATTN_ERR_UNSUPPORTED",
    "ATTN_ERR_WORKSPACE",
    "ATTN_F32",
    "ATTN_NOALLOC_SCRATCH_BYTES",
    "ATTN_OK",
    "LIB_PATH",
    "AttnError",
    "attn_abi_version",
    "attn_bwd",
    "attn_bwd_workspace_bytes",
    "attn_decode_paged",
    "attn_decode_paged_noalloc",
    "attn_decode_workspace_bytes",
    "attn_fwd",
    "attn_fwd_chunk",
    "attn_fwd_fp8",
    "attn_merge",
    "attn_quantize_fp8",
    "attn_status_str",
    "lib",
]
