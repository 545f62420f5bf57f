"""Prefill, decode and backward captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must give, bit for bit, what the same call gives
eagerly (the kernels are deterministic), with eager work and
synchronisations between the replays.  Cases: a multi-segment plan with the
look-back, the same with the separate prefix-scan kernel, packed documents
with an empty one, a decode step whose state is reset eagerly before
each replay, and the backward.  The eager prefill and decode results are
checked against the fp64 oracle."""
import numpy as np
import pytest

import causal_linear_attention_la_amd as la
import la_inputs
import oracle
from gpu_helpers import ErrAcc, log, to_dev, to_host

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    la.load()  # the HIP library must be present: no fallback
    la_inputs.build()
    oracle.build()
    yield


def _capture(fn):
    """fn() captured into a graph on a side stream (after one eager warm-up there)."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("case", ["lookback", "scan", "packed"])
def test_prefill_graph_replays_match_eager(case):
    import torch

    T, H, d = 3000, 4, 128
    cu = np.array([0, T], np.int32) if case != "packed" else np.array([0, 700, 700, 2300, T], np.int32)
    opts = dict(seg_len=256, force_scan=case == "scan")
    num_seqs = len(cu) - 1
    plan = la.la_prefill_plan(T, num_seqs, H, d, 64, la.LA_BF16, la.make_opts(**opts))
    assert plan["num_segments"] > 1 and plan["scan"] == (1 if case == "scan" else 0)
    log(f"  graph prefill {case}: plan {plan}")
    q, k, v = (la_inputs.normal(71, i, (T, H, d), "bf16", 1 / np.sqrt(d)) for i in range(3))
    qd, kd, vd, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(cu)
    o = torch.empty_like(qd)
    kv = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")

    def call():
        la.prefill(qd, kd, vd, cud, block=64, out=o, kv_state_out=kv, workspace=ws, **opts)

    call()
    torch.cuda.synchronize()
    o_ref, kv_ref = o.clone(), kv.clone()
    ref = oracle.recurrent(q, k, v, cu)
    ErrAcc().add(to_host(o_ref), ref[0]).check(False, f"graph {case} eager o")
    ErrAcc().add(to_host(kv_ref), ref[1]).check(True, f"graph {case} eager state")

    g = _capture(call)
    for r in range(REPLAYS):
        o.fill_(float("nan"))  # eager work between the replays
        kv.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"    replay {r}")
        assert torch.equal(o, o_ref), f"replay {r}: o differs from the eager call"
        assert torch.equal(kv, kv_ref), f"replay {r}: state differs from the eager call"


def test_decode_graph_replays_match_eager():
    import torch

    ns, H, d = 6, 4, 128
    S0 = la_inputs.decode_states(73, ns, H, d, 2 * d, 4096).reshape(ns, H, d, d)
    q, k, v = la_inputs.decode_step_inputs(74, 0, ns, H, d, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    S0d = to_dev(S0.copy())
    S = S0d.clone()
    o = torch.empty_like(qd)

    def call():
        la.decode(qd, kd, vd, S, out=o)

    call()
    torch.cuda.synchronize()
    o_ref, S_ref = o.clone(), S.clone()
    S_or = S0.astype(np.float64).reshape(ns * H, d, d).copy()
    o_or = oracle.decode_step(q.reshape(-1, d), k.reshape(-1, d), v.reshape(-1, d), S_or)
    ErrAcc().add(to_host(o_ref).reshape(-1, d), o_or).check(False, "graph decode eager o")
    ErrAcc().add(to_host(S_ref).reshape(-1, d, d), S_or).check(True, "graph decode eager state")

    S.copy_(S0d)
    g = _capture(call)  # (warm-up and capture each advance the state once more; reset below)
    for r in range(REPLAYS):
        S.copy_(S0d)  # eager reset of the state the step updates in place
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"    decode replay {r}")
        assert torch.equal(o, o_ref), f"replay {r}: o differs from the eager step"
        assert torch.equal(S, S_ref), f"replay {r}: state differs from the eager step"


def test_backward_graph_replays_match_eager():
    """The backward's passes (with the in-place transposes of segment states)
    captured together; every replay matches the eager call bit for bit (the
    eager gradients themselves are checked against the oracle elsewhere)."""
    import torch

    T, H, d = 2000, 2, 128
    cu = np.array([0, 900, T], np.int32)
    opts = dict(seg_len=256)
    q, k, v, dout = (la_inputs.normal(75, i, (T, H, d), "bf16", 1 / np.sqrt(d)) for i in range(4))
    qd, kd, vd, dod, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(dout), to_dev(cu)
    dko = to_dev(la_inputs.normal(75, 9, (2, H, d, d), "fp32", 0.01))
    outs = (torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd),
            torch.empty((2, H, d, d), dtype=torch.float32, device="cuda"))
    need = la.la_prefill_workspace_size_ex(T, 2, H, d, 64, la.LA_BF16, la.make_opts(**opts))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call():
        la.backward(qd, kd, vd, dod, cud, block=64, dkv_state_out=dko, workspace=ws, out=outs, **opts)

    call()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    g = _capture(call)
    for r in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"    backward replay {r}")
        for name, t, ref in zip(("dq", "dk", "dv", "dkv_in"), outs, refs):
            assert torch.equal(t, ref), f"replay {r}: {name} differs from the eager call"
