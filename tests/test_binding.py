"""The torch-level binding checks every tensor it is handed before any
pointer reaches the C ABI (no GPU needed: every call here must raise on the
host).  A host pointer, a wrong dtype, a short or non-contiguous buffer would
otherwise be read or written by the kernels."""
import pytest
import torch

import causal_linear_attention_la_amd as la

T, H, d = 64, 2, 16


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def cu(n=1, dtype=torch.int32):
    return torch.tensor([0] + [T] * n, dtype=dtype)


@pytest.mark.parametrize("change,exc", [
    (dict(k=torch.zeros(T, H, d)), TypeError),                          # k fp32, q bf16
    (dict(v=bf(T, H, d + 1)), ValueError),                              # wrong shape
    (dict(k=bf(T, d, H).transpose(1, 2)), ValueError),                  # not contiguous
    (dict(cu_seqlens=cu(dtype=torch.int64)), TypeError),                # int64 boundaries
    (dict(cu_seqlens=torch.tensor([0], dtype=torch.int32)), ValueError),  # no document
    (dict(kv_state_out=torch.zeros(1, H, d, d, dtype=torch.bfloat16)), TypeError),
    (dict(kv_state_out=torch.zeros(2, H, d, d)), ValueError),           # one document, two states
    (dict(kv_state_in=torch.zeros(1, H, d, d - 1)), ValueError),
    (dict(out=bf(T + 1, H, d)), ValueError),
    (dict(q=bf(T, H * d)), ValueError),                                 # not [T, H, d]
    (dict(workspace=torch.zeros(64, dtype=torch.uint8)[::2]), ValueError),
    (dict(), ValueError),                                               # every tensor valid but on the host
])
def test_prefill_rejects_before_launch(change, exc):
    a = dict(q=bf(T, H, d), k=bf(T, H, d), v=bf(T, H, d), cu_seqlens=cu())
    a.update(change)
    q, k, v, c = a.pop("q"), a.pop("k"), a.pop("v"), a.pop("cu_seqlens")
    with pytest.raises(exc):
        la.prefill(q, k, v, c, block=32, **a)


@pytest.mark.parametrize("change,exc", [
    (dict(kv_state=None), ValueError),
    (dict(kv_state=torch.zeros(2, H, d, d, dtype=torch.bfloat16)), TypeError),  # bf16 state
    (dict(kv_state=torch.zeros(1, H, d, d)), ValueError),                       # one sequence's state for two
    (dict(v=torch.zeros(2, H, d)), TypeError),
    (dict(out=bf(2, H, d)[:, :, :8]), ValueError),
    (dict(), ValueError),
])
def test_decode_rejects_before_launch(change, exc):
    a = dict(q=bf(2, H, d), k=bf(2, H, d), v=bf(2, H, d), kv_state=torch.zeros(2, H, d, d))
    a.update(change)
    with pytest.raises(exc):
        la.decode(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("kv_state"), **a)


@pytest.mark.parametrize("change,exc", [
    (dict(dout=torch.zeros(T, H, d)), TypeError),
    (dict(dkv_state_out=torch.zeros(1, H, d, d, dtype=torch.float64)), TypeError),
    (dict(out=(bf(T, H, d), bf(T, H, d), bf(T, H, d - 1), None)), ValueError),
    (dict(out=(bf(T, H, d), bf(T, H, d), bf(T, H, d), torch.zeros(1, H, d, 1))), ValueError),
    (dict(forward_workspace=torch.zeros(64, dtype=torch.uint8)[::2]), ValueError),
    (dict(), ValueError),
])
def test_backward_rejects_before_launch(change, exc):
    a = dict(q=bf(T, H, d), k=bf(T, H, d), v=bf(T, H, d), dout=bf(T, H, d), cu_seqlens=cu())
    a.update(change)
    with pytest.raises(exc):
        la.backward(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("dout"), a.pop("cu_seqlens"), block=32, **a)
