"""GPU parity of la_prefill_backward against the fp64 oracle's backward
(which is pinned to finite differences of the forward).

Cases: ragged packed documents (empty ones included) with and without
incoming states and final-state gradients, on both block loops (bf16 d = 128
and 64 on the gfx950 loop, bf16 block 32 and fp32 on the generic loop), with
segment splitting and the scan path (which in the reverse passes run over
documents read back to front), the document-piece work list, the 8192-token x 8-head workload in full, and
the 1M-token workload on the GPU in full, checked exactly on windows, and the
131072-token packed workload in full, two heads compared against the oracle."""
import numpy as np
import pytest

import causal_linear_attention_la_amd as la
import la_inputs
import oracle
from gpu_helpers import ErrAcc, as_f64, log, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    la.load()
    la_inputs.build()
    oracle.build()
    yield


def inputs(seed, T, H, d, dtype):
    scale = 1.0 / np.sqrt(d)
    q, k, v = (la_inputs.normal(seed, i, (T, H, d), dtype, scale) for i in range(3))
    dout = la_inputs.normal(seed, 8, (T, H, d), dtype, 1.0)
    return q, k, v, dout


def states(seed, tid, D, H, d, scale):
    return np.ascontiguousarray(la_inputs.normal(seed, tid, (D, H, d, d), "fp32", scale), dtype=np.float32)


def run(q, k, v, dout, cu, block, kv_in, dkv_out, **opts):
    import torch

    dq, dk, dv, dki = la.backward(to_dev(q), to_dev(k), to_dev(v), to_dev(dout), to_dev(np.asarray(cu, np.int32)),
                                  block=block, kv_state_in=None if kv_in is None else to_dev(kv_in),
                                  dkv_state_out=None if dkv_out is None else to_dev(dkv_out), **opts)
    torch.cuda.synchronize()
    return to_host(dq), to_host(dk), to_host(dv), to_host(dki)


def check(q, k, v, dout, cu, kv_in, dkv_out, got, fp32, what):
    ref = oracle.backward(q, k, v, dout, cu, kv_in=kv_in, dkv_out=dkv_out)
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        ErrAcc().add(g, r).check(fp32, f"{what} {name}")
    # dkv_in is a sum of fp32 outer products: held to the fp32 bound
    ErrAcc().add(got[3], ref[3]).check(True, f"{what} dkv_in")


CASES = [(d, block, dtype, opts, with_states)
         for d, block, dtype in ((128, 64, "bf16"), (64, 64, "bf16"), (128, 128, "bf16"), (128, 32, "bf16"),
                                 (32, 64, "fp32"))
         for opts in (dict(), dict(seg_len=2 * block, value_slices=2), dict(seg_len=block, force_scan=True),
                      dict(seg_len=max(128, 2 * block), work_list=2))
         for with_states in (False, True)]


@pytest.mark.parametrize("d,block,dtype,opts,with_states", CASES,
                         ids=[f"d{c[0]}-b{c[1]}-{c[2]}-{c[3]}-{'states' if c[4] else 'zero'}" for c in CASES])
def test_backward_against_oracle(d, block, dtype, opts, with_states):
    lens = [300, 0, 1, 700, 64, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H = int(cu[-1]), 3
    q, k, v, dout = inputs(111 + d, T, H, d, dtype)
    kv_in = states(112 + d, 7, len(lens), H, d, float(np.sqrt(2000)) / d) if with_states else None
    dkv_out = states(113 + d, 9, len(lens), H, d, 1.0) if with_states else None
    log(f"  backward d={d} block={block} {dtype} {opts} states={with_states}")
    got = run(q, k, v, dout, cu, block, kv_in, dkv_out, **opts)
    check(q, k, v, dout, cu, kv_in, dkv_out, got, dtype == "fp32", "backward")
    if with_states:
        # an empty document passes its final-state gradient straight to its incoming state
        for i, n in enumerate(lens):
            if n == 0:
                assert np.array_equal(got[3][i], dkv_out[i])


@pytest.mark.parametrize("slots", [2, 3])
def test_backward_tile_slots(slots):
    """All three passes (two of them over documents read back to front) with
    two and three tile slots in the block loop."""
    lens = [300, 0, 1, 700, 64, 0, 129, 1500]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 3, 128
    q, k, v, dout = inputs(131, T, H, d, "bf16")
    kv_in = states(132, 7, len(lens), H, d, float(np.sqrt(2000)) / d)
    dkv_out = states(133, 9, len(lens), H, d, 1.0)
    log(f"  backward slots={slots}")
    got = run(q, k, v, dout, cu, 64, kv_in, dkv_out, seg_len=1024, slots=slots)
    check(q, k, v, dout, cu, kv_in, dkv_out, got, False, f"backward slots {slots}")


@pytest.mark.parametrize("opts", [dict(seg_len=64), dict(seg_len=192), dict(seg_len=256, force_scan=True),
                                  dict(seg_len=128, value_slices=2)], ids=str)
@pytest.mark.parametrize("with_states", [False, True])
def test_backward_with_forward_states(opts, with_states):
    """The backward handed the forward's workspace (forward_states): the dq
    pass takes the forward's segment states, transposed, instead of its own.
    Against the oracle, and close to the backward computed from scratch."""
    import torch

    lens = [300, 0, 1, 700, 64, 0, 129, 1500]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 3, 128
    q, k, v, dout = inputs(151, T, H, d, "bf16")
    kv_in = states(152, 7, len(lens), H, d, float(np.sqrt(2000)) / d) if with_states else None
    dkv_out = states(153, 9, len(lens), H, d, 1.0) if with_states else None
    qd, kd, vd, dod, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(dout), to_dev(cu)
    kin = None if kv_in is None else to_dev(kv_in)
    dko = None if dkv_out is None else to_dev(dkv_out)
    need = la.la_prefill_workspace_size_ex(T, len(lens), H, d, 64, la.LA_BF16, la.make_opts(**opts))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    log(f"  backward with forward states {opts} states={with_states}")
    la.prefill(qd, kd, vd, cud, block=64, workspace=ws, kv_state_in=kin, **opts)
    got = la.backward(qd, kd, vd, dod, cud, block=64, kv_state_in=kin, dkv_state_out=dko, forward_workspace=ws, **opts)
    fresh = la.backward(qd, kd, vd, dod, cud, block=64, kv_state_in=kin, dkv_state_out=dko, **opts)
    torch.cuda.synchronize()
    got = tuple(to_host(x) for x in got)
    check(q, k, v, dout, cu, kv_in, dkv_out, got, False, "backward with forward states")
    ErrAcc().add(got[0], as_f64(to_host(fresh[0]))).check(False, "dq reused vs fresh")
    for a, b in zip(got[1:], fresh[1:]):
        assert np.array_equal(a, to_host(b)), "only the dq pass may change"


PAIR_CASES = [(128, dict()), (128, dict(seg_len=192)), (128, dict(seg_len=128, force_scan=True)),
              (128, dict(seg_len=256, value_slices=2)), (128, dict(seg_len=1024, value_slices=2, slots=3)),
              (128, dict(seg_len=1024, slots=3)), (128, dict(seg_len=384, work_list=2)), (64, dict(seg_len=128))]


@pytest.mark.parametrize("d,opts", PAIR_CASES, ids=[f"d{d}-{o}" for d, o in PAIR_CASES])
def test_paired_reverse_passes(d, opts):
    """With a workspace of la_prefill_backward_workspace_size bytes the dv and
    dk passes share one launch (la_prefill_pair_v2); with the forward's size
    they run one after the other.  Same kernels, same states: the gradients
    must agree bit for bit, and match the oracle."""
    import torch

    lens = [700, 0, 1, 1563, 64, 0, 437, 2100]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H = int(cu[-1]), 3
    q, k, v, dout = inputs(331, T, H, d, "bf16")
    kv_in = states(332, 7, len(lens), H, d, float(np.sqrt(300)) / d)
    dkv_out = states(333, 9, len(lens), H, d, 0.1)
    mo = la.make_opts(**opts)
    fwd_ws = la.la_prefill_workspace_size_ex(T, len(lens), H, d, 64, la.LA_BF16, mo)
    bwd_ws = la.la_prefill_backward_workspace_size(T, len(lens), H, d, 64, la.LA_BF16, mo)
    plan = la.la_prefill_plan(T, len(lens), H, d, 64, la.LA_BF16, mo)
    log(f"  paired {d} {opts} plan={plan} ws {fwd_ws} / {bwd_ws}")
    assert bwd_ws >= fwd_ws
    outs = []
    for nbytes in (fwd_ws, bwd_ws):
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        outs.append(run(q, k, v, dout, cu, 64, kv_in, dkv_out, workspace=ws, **opts))
    for name, a, b in zip(("dq", "dk", "dv", "dkv_in"), outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"paired {name} differs from sequential"
    check(q, k, v, dout, cu, kv_in, dkv_out, outs[1], False, f"paired d={d} {opts}")


def test_forward_states_are_claimed_once():
    """forward_states reuses the forward's segment states only while the
    workspace holds the stamp of a forward call on these very inputs, shapes
    and plan, and the first backward consumes it.  Checked three ways:
    (1) the states region is zeroed after the forward (the stamp stays): the
    first backward takes the zeros, as reuse must (the contents are the
    caller's precondition), and its dq is far from the truth, while a second
    backward on the same workspace computes its states and equals the fresh
    backward bit for bit; (2) a forward on other tensors of the same shape
    leaves a stamp that does not match; (3) a forward with another plan
    neither, even right after one with this plan; (4) a backward without
    forward_states clears the stamp of the states it overwrites."""
    import torch

    lens = [300, 0, 1, 700, 64, 0, 129, 1500]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 3, 128
    q, k, v, dout = inputs(161, T, H, d, "bf16")
    qd, kd, vd, dod, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(dout), to_dev(cu)
    opts = dict(seg_len=192)
    plan = la.la_prefill_plan(T, len(lens), H, d, 64, la.LA_BF16, la.make_opts(**opts))
    other = la.la_prefill_plan(T, len(lens), H, d, 64, la.LA_BF16, la.make_opts(seg_len=128))
    assert plan["num_segments"] > 2 and plan["packed"] == 0
    ws = torch.empty(max(plan["workspace_bytes"], other["workspace_bytes"]), dtype=torch.uint8, device="cuda")
    header = 256  # the workspace's stamp; the segment states follow it
    states = ws[header:header + (plan["num_segments"] - 1) * H * d * d * 4]
    fresh = [to_host(x) for x in la.backward(qd, kd, vd, dod, cud, block=64, **opts)[:3]]
    ref = oracle.backward(q, k, v, dout, cu)

    def bwd():
        got = la.backward(qd, kd, vd, dod, cud, block=64, forward_workspace=ws, **opts)
        torch.cuda.synchronize()
        return [to_host(x) for x in got[:3]]

    # (1) reuse happens once, and only once
    la.prefill(qd, kd, vd, cud, block=64, workspace=ws, **opts)
    states.zero_()
    first = bwd()
    e = ErrAcc().add(first[0], ref[0])
    log(f"    dq from zeroed reused states: rel_l2={e.rel_l2:.3e}")
    assert e.rel_l2 > 0.1, "the first backward must take the stamped workspace's states"
    second = bwd()
    for g, f in zip(second, fresh):
        assert np.array_equal(g, f), "a consumed stamp must not be reused"
    # (2) a forward on other tensors of the same shape
    q2, k2, v2 = (to_dev(x) for x in inputs(162, T, H, d, "bf16")[:3])
    la.prefill(q2, k2, v2, cud, block=64, workspace=ws, **opts)
    for g, f in zip(bwd(), fresh):
        assert np.array_equal(g, f), "states of other inputs must not be reused"
    # (3) a forward with another plan on the same workspace, after one with this plan
    la.prefill(qd, kd, vd, cud, block=64, workspace=ws, **opts)
    la.prefill(qd, kd, vd, cud, block=64, workspace=ws, seg_len=128)
    for g, f in zip(bwd(), fresh):
        assert np.array_equal(g, f), "states of another plan must not be reused"
    # (4) a backward without forward_states overwrites the states: its stamp goes too
    la.prefill(qd, kd, vd, cud, block=64, workspace=ws, **opts)
    la.backward(qd, kd, vd, dod, cud, block=64, workspace=ws, **opts)
    for g, f in zip(bwd(), fresh):
        assert np.array_equal(g, f), "states overwritten by a backward must not be reused"
    for name, g, r in zip(("dq", "dk", "dv"), second, ref[:3]):
        ErrAcc().add(g, r).check(False, f"second backward {name}")


def test_backward_prefill_8k_workload():
    w = la_inputs.prefill_inputs("prefill_8k")
    T, H, d = w["T"], w["H"], w["d"]
    dout = la_inputs.normal(la_inputs.WORKLOADS["prefill_8k"]["seed"], 8, (T, H, d), "bf16", 1.0)
    log(f"  backward prefill_8k T={T} H={H}")
    got = run(w["q"], w["k"], w["v"], dout, w["cu"], w["block"], None, None)
    check(w["q"], w["k"], w["v"], dout, w["cu"], None, None, got, False, "backward 8k")


def test_backward_long_1m_windows():
    """The 1M-token x 8-head workload's backward in full on the GPU, checked
    exactly on windows: the first tokens, a window across a segment end in
    the middle, and the last tokens.  For a window [a, b) the oracle takes
    the forward state before it (sum of k^T v over [0, a)) and the reverse
    state after it (sum of q^T dO over [b, T)) as boundary states and runs
    its backward on the window alone, which gives that window's dq, dk, dv
    of the whole sequence."""
    import torch

    w = la_inputs.prefill_inputs("long_1m")
    T, H, d = w["T"], w["H"], w["d"]
    q, k, v = w["q"], w["k"], w["v"]
    dout = la_inputs.normal(la_inputs.WORKLOADS["long_1m"]["seed"], 8, (T, H, d), "bf16", 1.0)
    plan = la.la_prefill_plan(T, 1, H, d, 64, la.LA_BF16)
    log(f"  backward long_1m plan={plan}")
    dq, dk, dv, _ = la.backward(to_dev(q), to_dev(k), to_dev(v), to_dev(dout), to_dev(w["cu"]), block=64,
                                want_dkv_in=False)
    torch.cuda.synchronize()
    n, L = 4096, plan["seg_len"]
    for a in (0, (plan["num_segments"] // 2) * L - n // 2, T - n):
        b = a + n
        kv_a = oracle.recurrent(q[:a], k[:a], v[:a], np.array([0, a], np.int32), want_o=False)[1] if a else None
        g_b = oracle.recurrent(q[b:], q[b:], dout[b:], np.array([0, T - b], np.int32), want_o=False)[1] \
            if b < T else None
        ref = oracle.backward(q[a:b], k[a:b], v[a:b], dout[a:b], np.array([0, n], np.int32), kv_in=kv_a,
                              dkv_out=g_b, want_dkv_in=False)
        for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
            ErrAcc().add(to_host(g[a:b]), r).check(False, f"long_1m window [{a}, {b}) {name}")
        log(f"    window [{a}, {b}) compared")


def test_backward_varlen_128k_heads():
    """The 131072-token x 64-head packed workload (20 documents) backward in
    full on the GPU; two heads compared in full against the oracle's backward
    run on those heads alone (heads are independent)."""
    import torch

    w = la_inputs.prefill_inputs("varlen_128k")
    T, H, d = w["T"], w["H"], w["d"]
    q, k, v, cu = w["q"], w["k"], w["v"], w["cu"]
    dout = la_inputs.normal(la_inputs.WORKLOADS["varlen_128k"]["seed"], 8, (T, H, d), "bf16", 1.0)
    plan = la.la_prefill_plan(T, len(cu) - 1, H, d, 64, la.LA_BF16)
    log(f"  backward varlen_128k docs={len(cu) - 1} plan={plan}")
    dq, dk, dv, dki = la.backward(to_dev(q), to_dev(k), to_dev(v), to_dev(dout), to_dev(cu), block=64)
    torch.cuda.synchronize()
    for h0 in (0, 37):
        sl = slice(h0, h0 + 2)
        part = [np.ascontiguousarray(x[:, sl]) for x in (q, k, v, dout)]
        ref = oracle.backward(*part, cu)
        for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
            ErrAcc().add(to_host(g[:, sl]), r).check(False, f"varlen heads {h0}..{h0 + 1} {name}")
        ErrAcc().add(to_host(dki[:, sl]), ref[3]).check(True, f"varlen heads {h0}..{h0 + 1} dkv_in")
        log(f"    heads {h0}..{h0 + 1} compared")


def test_backward_rejects_aliasing():
    import torch

    T, H, d = 128, 2, 64
    q, k, v, dout = (to_dev(x) for x in inputs(121, T, H, d, "bf16"))
    cu = to_dev(np.array([0, T], np.int32))
    with pytest.raises(la.LAError):
        la_dq = q  # gradient written over an input
        st = la.la_prefill_backward(la._ptr(q), la._ptr(k), la._ptr(v), la._ptr(dout), la._ptr(cu), H, d, 64, None,
                                    None, la._ptr(la_dq), la._ptr(torch.empty_like(q)), la._ptr(torch.empty_like(q)),
                                    None, 1, T, la.LA_BF16, None, 0, None, None)
        if st != la.LA_OK:
            raise la.LAError(st, "la_prefill_backward")
