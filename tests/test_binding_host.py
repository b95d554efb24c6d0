"""Host-side argument checks of the Python binding, on the CPU: shape errors must be raised
before anything reaches the library (the C ABI cannot see buffer sizes, so a short output
passed through would be written past its end).  The device checks are stood in for by a
dtype/contiguity check and the library by a stub that fails the test if it is called."""

import pytest
import torch

import online_softmax_attn_amd.binding as binding


class _NoLibrary:
    def __getattr__(self, name):
        if name.endswith("_workspace_bytes"):
            return lambda *a: 1 << 20
        raise AssertionError(f"{name} was reached with invalid arguments")


@pytest.fixture
def host_binding(monkeypatch):
    def check_host(name, t, dtype=None):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a tensor")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    monkeypatch.setattr(binding, "_check_dev", check_host)
    monkeypatch.setattr(binding, "lib", lambda: _NoLibrary())
    return binding


def _decode_args(B=2, H=4, Hkv=2, d=128, nb=6):
    bf = torch.bfloat16
    q = torch.zeros(B, H, d, dtype=bf)
    kc = torch.zeros(nb, Hkv, 16, d, dtype=bf)
    vc = torch.zeros(nb, Hkv, 16, d, dtype=bf)
    table = torch.zeros(B, 3, dtype=torch.int32)
    return q, kc, vc, table


@pytest.mark.parametrize("shape", [(2, 4, 64), (2, 3, 128), (1, 4, 128), (8, 128)])
def test_decode_rejects_an_output_of_the_wrong_shape(host_binding, shape):
    q, kc, vc, table = _decode_args()
    out = torch.zeros(shape, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must be"):
        host_binding.attn_decode_paged(q, kc, vc, table, [10, 20], max_seq_len=48, out=out)


@pytest.mark.parametrize("shape", [(2,), (2, 3), (4, 2), (2, 4, 1)])
def test_decode_rejects_an_lse_of_the_wrong_shape(host_binding, shape):
    q, kc, vc, table = _decode_args()
    out = torch.zeros(2, 4, 128, dtype=torch.bfloat16)
    lse = torch.zeros(shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="lse must be"):
        host_binding.attn_decode_paged(q, kc, vc, table, [10, 20], max_seq_len=48, out=out, lse=lse)


def test_prefill_rejects_outputs_of_the_wrong_shape(host_binding):
    bf = torch.bfloat16
    q, k, v = (torch.zeros(1, 2, 64, 128, dtype=bf) for _ in range(3))
    with pytest.raises(ValueError, match="out must be"):
        host_binding.attn_fwd(q, k, v, out=torch.zeros(1, 2, 63, 128, dtype=bf))
    with pytest.raises(ValueError, match="lse must be"):
        host_binding.attn_fwd(q, k, v, lse=torch.zeros(1, 2, 65, dtype=torch.float32))
