"""Thin ctypes binding of libattn.so (include/attn.h).

The functions carry the C entry points' names.  They only marshal arguments: check
tensor dtypes, devices, shapes and contiguity, allocate outputs/workspace with torch when
the caller did not pass them, pass raw device pointers and torch's current HIP stream, and
raise on a non-OK status.  Every step of the attention itself runs in the HIP kernels; if
the library is not built this module raises instead of computing anything another way.
"""

from __future__ import annotations

import ctypes
import functools
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_LAUNCH = range(5)
ATTN_F32, ATTN_BF16 = 0, 1
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20  # include/attn.h: the no-alloc decode's scratch array

# name -> (restype, argtypes), exactly the declarations of include/attn.h
_P = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "attn_fwd": (_I, [_I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                      _P]),
    "attn_fwd_chunk": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                            ctypes.c_float, _P]),
    "attn_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "attn_bwd": (
        _I,
        [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
         _P, ctypes.c_size_t, _P],
    ),
    "attn_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_decode_paged": (
        _I,
        [_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
         _P, ctypes.c_size_t, _P],
    ),
    "attn_decode_paged_noalloc": (
        _I,
        [_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
         _P],
    ),
    "attn_quantize_fp8": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "attn_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                          ctypes.c_float, _P]),
    "attn_merge": (_I, [_I, _P, _P, _P, _P, _I, ctypes.c_int64, _I, _P]),
    "attn_status_str": (ctypes.c_char_p, [_I]),
    "attn_abi_version": (_I, []),
}
# the measurement kernels, exactly the declarations of include/attn_probe.h
PROBE_SIGNATURES = {
    "attn_probe_mfma": (_I, [_I, _I, _I, _P, _P]),
    "attn_probe_exp": (_I, [_I, _I, _P, _P]),
    "attn_probe_read": (_I, [_P, ctypes.c_size_t, _I, _P, _P]),
    "attn_probe_read_pages": (_I, [_P, _I, _P, _I, _I, _P, _P]),
}
ATTN_PROBE_THREADS = 256

_lib = None


class AttnError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {attn_status_str(status)} ({status})")


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m online_softmax_attn_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in {**SIGNATURES, **PROBE_SIGNATURES}.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def attn_status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def attn_abi_version() -> int:
    return int(lib().attn_abi_version())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _on_stream(fn):
    """Run an entry point with its `stream` argument (a torch.cuda.Stream or a raw hipStream_t
    handle) as torch's current stream, so that everything the binding allocates for the call
    (outputs, workspaces, uploaded lengths) belongs to the stream the kernels run on: the
    caching allocator then never hands that memory to other work while the kernels still
    use it."""

    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, stream=None, **kwargs)
        ts = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(ts):
            return fn(*args, stream=ts, **kwargs)

    return wrapper


def _check_dev(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")


_DT = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}


def _lengths(seq_lens, batch, limit, device, name="seq_lens"):
    """Lengths as a device int32 tensor.

    A host sequence is checked (batch entries, each in [1, limit]) before upload.  A device
    int32 tensor is passed through unchecked (reading it back would synchronise the
    stream); its range is then the caller's precondition, as in the C ABI.
    """
    if seq_lens is None:
        return None
    if isinstance(seq_lens, torch.Tensor) and seq_lens.is_cuda:
        if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous() or seq_lens.numel() != batch:
            raise ValueError(f"{name} on the device must be contiguous int32 with {batch} entries")
        return seq_lens
    host = torch.as_tensor(seq_lens).to(torch.int64).reshape(-1)
    if host.numel() != batch:
        raise ValueError(f"{name} must have {batch} entries")
    if int(host.min()) < 1 or int(host.max()) > limit:
        raise ValueError(f"{name} must lie in [1, {limit}]")
    return host.to(torch.int32).to(device)


def _kv_heads(q, k, v):
    """K/V head count of q [B, H, n, d] against k, v [B, H_kv, n, d] (H a multiple of H_kv)."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, H, n, d]; k and v one shape [B, H_kv, n, d]")
    B, H, n, d = q.shape
    Hkv = int(k.shape[1])
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, n, d) or Hkv < 1 or H % Hkv:
        raise ValueError("k, v must be [B, H_kv, n, d] with H a multiple of H_kv")
    return Hkv


@_on_stream
def attn_fwd(q, k, v, *, causal=False, window=0, scale=None, seq_lens=None, out=None,
             lse=None, return_lse=False, stream=None):
    """Prefill attention: q [B, H, n, d], k and v [B, H_kv, n, d] (d in {64, 128}, fp32 or
    bf16).

    seq_lens: optional per-batch lengths (host sequence or device int32 tensor); rows past
    a length are padding (output 0, lse -inf).  window > 0 (with causal) limits query i to
    keys i - window < j <= i.  Returns o, or (o, lse) with return_lse.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t)
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    Hkv = _kv_heads(q, k, v)
    B, H, n, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out, q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must be [B, H, n, d]")
    if lse is None and return_lse:
        lse = torch.empty(B, H, n, dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if lse.shape != (B, H, n):
            raise ValueError("lse must be [B, H, n]")
    lens = _lengths(seq_lens, B, n, q.device)
    st = lib().attn_fwd(_DT[q.dtype], q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr() if lse is not None else None,
                        lens.data_ptr() if lens is not None else None,
                        B, H, Hkv, n, d, int(bool(causal)), int(window), float(scale),
                        _stream(stream))
    if st != ATTN_OK:
        raise AttnError("attn_fwd", st)
    return (out, lse) if return_lse else out


@_on_stream
def attn_fwd_chunk(q, k, v, q_start, *, causal=False, window=0, scale=None, out=None,
                   lse=None, return_lse=False, stream=None):
    """A chunk of queries against a longer key sequence (bf16, d in {64, 128}): q [B, H, n_q, d] are
    positions q_start .. q_start + n_q - 1 of the sequence whose keys and values are
    k, v [B, H_kv, n_kv, d]; the causal mask and the window count those positions.
    Returns o, or (o, lse) with return_lse."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.bfloat16)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, H, n_q, d]; k and v one shape [B, H_kv, n_kv, d]")
    B, H, n_q, d = q.shape
    Hkv, n_kv = int(k.shape[1]), int(k.shape[2])
    if k.shape[0] != B or k.shape[3] != d or Hkv < 1 or H % Hkv:
        raise ValueError("k, v must be [B, H_kv, n_kv, d] with H a multiple of H_kv")
    if not 0 <= int(q_start) <= n_kv - n_q:
        raise ValueError("the chunk must lie inside the key sequence: 0 <= q_start <= n_kv - n_q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out, torch.bfloat16)
    if out.shape != q.shape:
        raise ValueError("out must be [B, H, n_q, d]")
    if lse is None and return_lse:
        lse = torch.empty(B, H, n_q, dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if lse.shape != (B, H, n_q):
            raise ValueError("lse must be [B, H, n_q]")
    st = lib().attn_fwd_chunk(ATTN_BF16, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              out.data_ptr(), lse.data_ptr() if lse is not None else None,
                              B, H, Hkv, n_q, n_kv, int(q_start), d, int(bool(causal)),
                              int(window), float(scale), _stream(stream))
    if st != ATTN_OK:
        raise AttnError("attn_fwd_chunk", st)
    return (out, lse) if return_lse else out


@_on_stream
def attn_merge(o_parts, lse_parts, *, out=None, lse=None, return_lse=False, stream=None):
    """Attention over the union of disjoint key sets from each set's (o, lse).

    o_parts: [S, ..., d] (bf16 or fp32, d in {64, 128}), the S parts stacked on the first
    dimension; lse_parts: fp32 [S, ...] with the same leading shape (-inf where a part admits
    no key of the row).  Returns o [..., d], or (o, lse) with return_lse.
    """
    _check_dev("o_parts", o_parts)
    _check_dev("lse_parts", lse_parts, torch.float32)
    if o_parts.dtype not in _DT:
        raise ValueError("o_parts must be float32 or bfloat16")
    if o_parts.dim() < 2 or tuple(lse_parts.shape) != tuple(o_parts.shape[:-1]):
        raise ValueError("o_parts must be [S, ..., d] and lse_parts [S, ...]")
    S, d = int(o_parts.shape[0]), int(o_parts.shape[-1])
    rows = o_parts.numel() // (S * d) if S * d else 0
    if out is None:
        out = torch.empty(o_parts.shape[1:], dtype=o_parts.dtype, device=o_parts.device)
    _check_dev("out", out, o_parts.dtype)
    if tuple(out.shape) != tuple(o_parts.shape[1:]):
        raise ValueError("out must be o_parts.shape[1:]")
    if lse is None and return_lse:
        lse = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=o_parts.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != tuple(lse_parts.shape[1:]):
            raise ValueError("lse must be lse_parts.shape[1:]")
    st = lib().attn_merge(_DT[o_parts.dtype], o_parts.data_ptr(), lse_parts.data_ptr(),
                          out.data_ptr(), lse.data_ptr() if lse is not None else None, S, rows,
                          d, _stream(stream))
    if st != ATTN_OK:
        raise AttnError("attn_merge", st)
    return (out, lse) if return_lse else out


def attn_bwd_workspace_bytes(batch, heads, seq_len) -> int:
    return int(lib().attn_bwd_workspace_bytes(batch, heads, seq_len))


@_on_stream
def attn_bwd(q, k, v, o, dout, lse, *, causal=False, window=0, scale=None, seq_lens=None,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) in fp32 of sum(o * dout), recomputing the weights from lse.

    q, o, dout: bf16 [B, H, n, 128]; k, v: bf16 [B, H_kv, n, 128]; lse: fp32 [B, H, n] from
    attn_fwd(return_lse=True) with the same mask, window, lengths and scale.  dk and dv have
    the shape of k (a shared K/V head gets the sum over its query heads).
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_dev(name, t, torch.bfloat16)
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    Hkv = _kv_heads(q, k, v)
    B, H, n, d = q.shape
    _check_dev("lse", lse, torch.float32)
    if lse.shape != (B, H, n):
        raise ValueError("lse must be [B, H, n]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for name, t, shape in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, k.shape)):
        if t is None:
            t = torch.empty(shape, dtype=torch.float32, device=q.device)
        _check_dev(name, t, torch.float32)
        if t.shape != shape:
            raise ValueError(f"{name} must be {tuple(shape)}")
        outs.append(t)
    need = attn_bwd_workspace_bytes(B, H, n)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_dev("workspace", workspace)
    lens = _lengths(seq_lens, B, n, q.device)
    st = lib().attn_bwd(ATTN_BF16, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                        dout.data_ptr(), lse.data_ptr(), lens.data_ptr() if lens is not None else None,
                        outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), B, H, Hkv, n,
                        d, int(bool(causal)), int(window), float(scale), workspace.data_ptr(),
                        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != ATTN_OK:
        raise AttnError("attn_bwd", st)
    return tuple(outs)


def attn_decode_workspace_bytes(batch, heads, head_dim, max_seq_len, kv_split=0, *,
                                kv_heads=None, window=0) -> int:
    kv_heads = heads if kv_heads is None else kv_heads
    return int(lib().attn_decode_workspace_bytes(batch, heads, kv_heads, head_dim, max_seq_len,
                                                 window, kv_split))


@_on_stream
def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len, window=0,
                      scale=None, kv_split=0, out=None, lse=None, return_lse=False,
                      workspace=None, stream=None):
    """One bf16 query per sequence ([B, H, d]) against a paged cache [blocks, H_kv, 16, d]
    (H a multiple of H_kv).  window > 0 admits only each sequence's last `window` tokens."""
    _check_dev("q", q, torch.bfloat16)
    _check_dev("k_cache", k_cache, torch.bfloat16)
    _check_dev("v_cache", v_cache, torch.bfloat16)
    _check_dev("block_table", block_table, torch.int32)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, H, d]; caches [num_blocks, H_kv, block_size, d]")
    B, H, d = q.shape
    nb, Hkv, bs, dc = k_cache.shape
    if Hkv < 1 or H % Hkv or dc != d:
        raise ValueError("cache heads must divide the query heads; head_dim must match q")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    if seq_lens is None:
        raise ValueError("seq_lens is required for decode")
    lens = _lengths(seq_lens, B, max_seq_len, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out, torch.bfloat16)
    if tuple(out.shape) != (B, H, d):
        raise ValueError("out must be [B, H, d]")
    if lse is None and return_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, H):
            raise ValueError("lse must be [B, H]")
    need = attn_decode_workspace_bytes(B, H, d, max_seq_len, kv_split, kv_heads=Hkv,
                                       window=window)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().attn_decode_paged(
        ATTN_BF16, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        lens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, H, Hkv, d, bs, nb, int(block_table.shape[1]), int(max_seq_len), int(window),
        float(scale), int(kv_split), workspace.data_ptr(), ws_bytes, _stream(stream))
    if st != ATTN_OK:
        raise AttnError("attn_decode_paged", st)
    return (out, lse) if return_lse else out


@_on_stream
def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len, out,
                              window=0, scale=None, kv_split=0, lse=None, stream=None):
    """attn_decode_paged without a workspace: the library's fixed per-GPU scratch array holds
    the split partials (ATTN_NOALLOC_SCRATCH_BYTES; larger requests raise AttnError with
    ATTN_ERR_WORKSPACE).  `out` (and `lse`, if wanted) must be given; `seq_lens` must be a
    device int32 tensor, so the call allocates nothing.  Overlapping calls on one GPU race."""
    for name, t, dt in (("q", q, torch.bfloat16), ("k_cache", k_cache, torch.bfloat16),
                        ("v_cache", v_cache, torch.bfloat16), ("block_table", block_table, torch.int32),
                        ("out", out, torch.bfloat16)):
        _check_dev(name, t, dt)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, H, d]; caches [num_blocks, H_kv, block_size, d]")
    B, H, d = q.shape
    nb, Hkv, bs, dc = k_cache.shape
    if Hkv < 1 or H % Hkv or dc != d:
        raise ValueError("cache heads must divide the query heads; head_dim must match q")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    if tuple(out.shape) != (B, H, d):
        raise ValueError("out must be [B, H, d]")
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, H):
            raise ValueError("lse must be [B, H]")
    if not (isinstance(seq_lens, torch.Tensor) and seq_lens.is_cuda):
        raise ValueError("seq_lens must be a device int32 tensor (an upload would allocate)")
    lens = _lengths(seq_lens, B, max_seq_len, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().attn_decode_paged_noalloc(
        ATTN_BF16, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        lens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, H, Hkv, d, bs, nb, int(block_table.shape[1]), int(max_seq_len), int(window),
        float(scale), int(kv_split), _stream(stream))
    if st != ATTN_OK:
        raise AttnError("attn_decode_paged_noalloc", st)
    return out


# --------------------------------------------------------------------------- FP8 E4M3
FP8_BLOCK = 64  # rows per quantisation block (one fp32 scale each)


@_on_stream
def attn_quantize_fp8(x, *, seq_lens=None, transpose=False, out=None, scales=None, stream=None):
    """E4M3 codes (uint8) and fp32 block scales of a bf16 [B, H, n, 128] tensor.

    transpose=False: codes [B, H, n, 128]; transpose=True: [B, H, 128, n_pad] with
    n_pad = 64 * ceil(n / 64) (the V layout attn_fwd_fp8 reads).  scales: [B, H, ceil(n/64)].
    Returns (codes, scales).
    """
    _check_dev("x", x, torch.bfloat16)
    if x.dim() != 4:
        raise ValueError("x must be [B, H, n, d]")
    B, H, n, d = x.shape
    nb = -(-n // FP8_BLOCK)
    shape = (B, H, d, nb * FP8_BLOCK) if transpose else (B, H, n, d)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(B, H, nb, dtype=torch.float32, device=x.device)
    _check_dev("out", out, torch.uint8)
    _check_dev("scales", scales, torch.float32)
    if tuple(out.shape) != shape or tuple(scales.shape) != (B, H, nb):
        raise ValueError(f"out must be {shape} and scales {(B, H, nb)}")
    lens = _lengths(seq_lens, B, n, x.device)
    st = lib().attn_quantize_fp8(x.data_ptr(), out.data_ptr(), scales.data_ptr(),
                                 lens.data_ptr() if lens is not None else None, B, H, n, d,
                                 int(bool(transpose)), _stream(stream))
    if st != ATTN_OK:
        raise AttnError("attn_quantize_fp8", st)
    return out, scales


@_on_stream
def attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, *, causal=False, scale=None,
                 seq_lens=None, out=None, lse=None, return_lse=False, stream=None):
    """Prefill attention on E4M3 operands from attn_quantize_fp8 (q, k row-major, v
    transposed); bf16 output [B, H, n, 128]."""
    for name, t in (("q8", q8), ("k8", k8), ("vt8", vt8)):
        _check_dev(name, t, torch.uint8)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check_dev(name, t, torch.float32)
    if q8.dim() != 4 or k8.dim() != 4 or vt8.dim() != 4:
        raise ValueError("q8, k8 must be [B, H, n, d]; vt8 [B, H_kv, d, n_pad]")
    B, H, n, d = q8.shape
    Hkv = int(k8.shape[1])
    nb = -(-n // FP8_BLOCK)
    if tuple(k8.shape) != (B, Hkv, n, d) or Hkv < 1 or H % Hkv:
        raise ValueError("k8 must be [B, H_kv, n, d] with H a multiple of H_kv")
    if tuple(vt8.shape) != (B, Hkv, d, nb * FP8_BLOCK):
        raise ValueError("vt8 must be [B, H_kv, d, 64 * ceil(n / 64)]")
    if (tuple(q_scale.shape) != (B, H, nb) or tuple(k_scale.shape) != (B, Hkv, nb)
            or tuple(v_scale.shape) != (B, Hkv, nb)):
        raise ValueError("scales must be [B, heads, ceil(n / 64)]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(B, H, n, d, dtype=torch.bfloat16, device=q8.device)
    _check_dev("out", out, torch.bfloat16)
    if tuple(out.shape) != (B, H, n, d):
        raise ValueError("out must be [B, H, n, d]")
    if lse is None and return_lse:
        lse = torch.empty(B, H, n, dtype=torch.float32, device=q8.device)
    if lse is not None:
        _check_dev("lse", lse, torch.float32)
        if lse.shape != (B, H, n):
            raise ValueError("lse must be [B, H, n]")
    lens = _lengths(seq_lens, B, n, q8.device)
    st = lib().attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), q_scale.data_ptr(),
                            k_scale.data_ptr(), v_scale.data_ptr(), out.data_ptr(),
                            lse.data_ptr() if lse is not None else None,
                            lens.data_ptr() if lens is not None else None, B, H, Hkv, n, d,
                            int(bool(causal)), float(scale), _stream(stream))
    if st != ATTN_OK:
        raise AttnError("attn_fwd_fp8", st)
    return (out, lse) if return_lse else out


# ---- measurement kernels (include/attn_probe.h)

def _raise(func, status):
    if status != ATTN_OK:
        raise AttnError(func, status)


def _probe_out(n, dtype, device, out):
    if out is None:
        return torch.empty(n, dtype=dtype, device=device)
    _check_dev("out", out, dtype)
    if out.numel() < n:
        raise ValueError(f"out holds {out.numel()} values, the probe writes {n}")
    return out


@_on_stream
def attn_probe_mfma(fp8, blocks, iters, *, device="cuda", out=None, stream=None):
    """Matrix-core rate probe; returns out (float32[blocks * 4], each 1024 * iters for bf16,
    4096 * iters for fp8)."""
    out = _probe_out(blocks * (ATTN_PROBE_THREADS // 64), torch.float32, device, out)
    _raise("attn_probe_mfma", lib().attn_probe_mfma(int(bool(fp8)), blocks, iters,
                                                    _P(out.data_ptr()), _stream(stream)))
    return out


@_on_stream
def attn_probe_exp(blocks, iters, *, device="cuda", out=None, stream=None):
    """v_exp_f32 rate probe; returns out (float32[blocks * 256])."""
    out = _probe_out(blocks * ATTN_PROBE_THREADS, torch.float32, device, out)
    _raise("attn_probe_exp", lib().attn_probe_exp(blocks, iters, _P(out.data_ptr()),
                                                  _stream(stream)))
    return out


@_on_stream
def attn_probe_read(src, blocks, *, out=None, stream=None):
    """Streaming-read probe over the bytes of a contiguous device tensor (a multiple of
    4096 bytes); returns the per-thread wrapping word sums (int32 view of uint32)."""
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    out = _probe_out(blocks * ATTN_PROBE_THREADS, torch.int32, src.device, out)
    nbytes = src.numel() * src.element_size()
    _raise("attn_probe_read", lib().attn_probe_read(_P(src.data_ptr()), nbytes, blocks,
                                                      _P(out.data_ptr()), _stream(stream)))
    return out


@_on_stream
def attn_probe_read_pages(pool, order, blocks, *, out=None, stream=None):
    """Paged-read probe: the 4 KiB pages of `pool` (contiguous device tensor) in the order
    of `order` (device int32); returns the per-thread wrapping word sums."""
    if not (pool.is_cuda and pool.is_contiguous()):
        raise ValueError("pool must be a contiguous device tensor")
    _check_dev("order", order, torch.int32)
    nbytes = pool.numel() * pool.element_size()
    if nbytes % 4096:
        raise ValueError("pool must hold whole 4 KiB pages")
    out = _probe_out(blocks * ATTN_PROBE_THREADS, torch.int32, pool.device, out)
    _raise("attn_probe_read_pages",
           lib().attn_probe_read_pages(_P(pool.data_ptr()), nbytes // 4096, _P(order.data_ptr()),
                                       order.numel(), blocks, _P(out.data_ptr()), _stream(stream)))
    return out
