"""la_prefill_noalloc against la_prefill (through the C ABI).

The allocation-free entry point runs the same plan and kernels as la_prefill
with its segment states in the library's static device array instead of a
caller's workspace, so its outputs must equal la_prefill's bit for bit.  Two
calls in a row, the second on a smaller input with packed documents (the
array keeps the first call's contents); the outputs are also checked against
the fp64 oracle at the bf16 tolerances.  (A shape whose plan needs more than
the array holds is refused on the host: tests/test_abi.py.)"""
import ctypes

import numpy as np
import pytest

import causal_linear_attention_la_amd as la
import la_inputs
import oracle
from gpu_helpers import ErrAcc, log, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    la.load()
    la_inputs.build()
    oracle.build()
    yield


def P(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def both(seed, T, H, d, cu):
    import torch

    scale = 1.0 / np.sqrt(d)
    q, k, v = (la_inputs.normal(seed, i, (T, H, d), "bf16", scale) for i in range(3))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    cud = to_dev(np.asarray(cu, dtype=np.int32))
    ns = len(cu) - 1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    plan = la.la_prefill_plan(T, ns, H, d, 64, la.LA_BF16)
    log(f"  noalloc T={T} H={H} d={d} docs={ns} plan={plan}")
    assert plan["workspace_bytes"] > 0, "the case must use a workspace"
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
    o1, o2 = torch.empty_like(qd), torch.full_like(qd, float("nan"))
    kv1 = torch.empty((ns, H, d, d), dtype=torch.float32, device="cuda")
    kv2 = torch.full_like(kv1, float("nan"))
    st = la.la_prefill(P(qd), P(kd), P(vd), P(o1), P(cud), H, d, 64, P(kv1), ns, T, la.LA_BF16, P(ws),
                       plan["workspace_bytes"], stream)
    assert st == la.LA_OK, la.status_string(st)
    st = la.la_prefill_noalloc(P(qd), P(kd), P(vd), P(o2), P(cud), H, d, 64, P(kv2), ns, T, la.LA_BF16, stream)
    assert st == la.LA_OK, la.status_string(st)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(o1), to_host(o2)), "o differs from la_prefill's"
    assert np.array_equal(to_host(kv1), to_host(kv2)), "kv_state differs from la_prefill's"
    o_ref, kv_ref = oracle.recurrent(q, k, v, np.asarray(cu, dtype=np.int32))
    ErrAcc().add(to_host(o2), o_ref).check(False, "noalloc o")
    ErrAcc().add(to_host(kv2), kv_ref).check(False, "noalloc kv_state")


def test_noalloc_matches_prefill_twice():
    both(311, 8192, 8, 128, [0, 8192])                  # 16 segments x 2 slices, 8 MiB of states
    both(312, 4096, 4, 128, [0, 1500, 1500, 4096])      # smaller, packed, an empty document
