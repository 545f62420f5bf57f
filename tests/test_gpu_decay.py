"""GPU parity of the decayed variant (la_prefill_decay, la_decode_decay)
against the fp64 oracle's decayed forms (through the C ABI).

The reading of the decay the pages name but never define: per head h,
S_t = lambda_h S_{t-1} + k_t^T v_t and o_t = q_t . S_t.  Cases: every
(d, block, dtype) on ragged packed documents with incoming states and
per-head factors from 0 to 1; segment splitting with the look-back and with
the scan (segment states faded across segments); the document-piece work
list; two and three tile slots on the 64-column loop; lambda = 1 equal bit for
bit to the plain prefill on the gfx950 loop; chunked prefill continuing
across calls; and decode steps continuing a decayed prefill."""
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


def lam_for(H, seed):
    base = np.array([0.0, 0.5, 0.9, 0.99, 0.999, 1.0, 0.25, 0.97], dtype=np.float32)
    return np.roll(base, seed)[:H].copy()


def run(q, k, v, cu, block, lam, kv_in=None, **opts):
    import torch

    o, kv = la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(np.asarray(cu, np.int32)), block=block,
                       decay=to_dev(lam), kv_state_in=None if kv_in is None else to_dev(kv_in), **opts)
    torch.cuda.synchronize()
    return to_host(o), to_host(kv)


def check(q, k, v, cu, lam, kv_in, o, kv, fp32, what):
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu, kv_in=kv_in, decay=lam.astype(np.float64))
    ErrAcc().add(o, o_ref).check(fp32, f"{what} o")
    ErrAcc().add(kv, kv_ref).check(fp32, f"{what} kv_state")


SUPPORTED = [(d, b, dt) for d in (16, 32, 64, 128) for b in (32, 64, 128) for dt in ("bf16", "fp32")
             if not (dt == "fp32" and d >= 64 and b == 128)]


@pytest.mark.parametrize("d,block,dtype", SUPPORTED, ids=[f"d{d}-b{b}-{t}" for d, b, t in SUPPORTED])
def test_decay_shapes(d, block, dtype):
    lens = [1, 0, 199, 411, 389]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H = int(cu[-1]), 4
    scale = 1.0 / np.sqrt(d)
    q, k, v = (la_inputs.normal(201 + d + block, i, (T, H, d), dtype, scale) for i in range(3))
    kv_in = np.ascontiguousarray(la_inputs.normal(202, 7, (len(lens), H, d, d), "fp32", float(np.sqrt(500)) / d),
                                 dtype=np.float32)
    lam = lam_for(H, d + block)
    log(f"  decay d={d} block={block} {dtype} lambda={lam.tolist()}")
    o, kv = run(q, k, v, cu, block, lam, kv_in)
    check(q, k, v, cu, lam, kv_in, o, kv, dtype == "fp32", f"decay d{d} b{block} {dtype}")


SPLITS = [dict(seg_len=64, value_slices=1), dict(seg_len=64, value_slices=2, force_scan=True),
          dict(seg_len=192, value_slices=2), dict(seg_len=128, value_slices=1, force_scan=True),
          dict(seg_len=256, work_list=2), dict(seg_len=192, value_slices=2, work_list=2),
          dict(seg_len=1024, value_slices=2, slots=3), dict(seg_len=1024, value_slices=1),
          dict(seg_len=64, variant=1), dict(seg_len=128, variant=1, force_scan=True)]


@pytest.mark.parametrize("opts", SPLITS, ids=[str(s) for s in SPLITS])
def test_decay_segments(opts):
    """Segment states faded across the segments between them (look-back),
    chained by the scan, or summed over a document's pieces."""
    lens = [700, 0, 1, 1563, 64, 0, 437]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 3, 128
    scale = 1.0 / np.sqrt(d)
    q, k, v = (la_inputs.normal(211, i, (T, H, d), "bf16", scale) for i in range(3))
    kv_in = np.ascontiguousarray(la_inputs.normal(212, 7, (len(lens), H, d, d), "fp32", float(np.sqrt(500)) / d),
                                 dtype=np.float32)
    lam = np.array([0.995, 0.9, 0.999], dtype=np.float32)
    plan = la.la_prefill_plan(T, len(lens), H, d, 64, la.LA_BF16, la.make_opts(**opts))
    log(f"  decay {opts} plan={plan}")
    o, kv = run(q, k, v, cu, 64, lam, kv_in, **opts)
    check(q, k, v, cu, lam, kv_in, o, kv, False, f"decay {opts}")


@pytest.mark.parametrize("opts", [dict(), dict(seg_len=192, value_slices=2), dict(seg_len=128, force_scan=True),
                                  dict(seg_len=256, work_list=2)], ids=str)
def test_decay_one_is_plain(opts):
    """lambda = 1 on the gfx950 loop: bit for bit the plain prefill (the
    factors are all 1 or 0, and the per-block arithmetic is otherwise the same)."""
    lens = [300, 0, 1, 1200, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 128
    scale = 1.0 / np.sqrt(d)
    q, k, v = (la_inputs.normal(221, i, (T, H, d), "bf16", scale) for i in range(3))
    o1, kv1 = run(q, k, v, cu, 64, np.ones(H, np.float32), **opts)
    import torch

    o2, kv2 = la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(cu), block=64, **opts)
    torch.cuda.synchronize()
    assert np.array_equal(o1, to_host(o2)) and np.array_equal(kv1, to_host(kv2))


def test_decay_chunked_prefill_and_decode():
    """A decayed prefill cut in three calls, each resuming from the previous
    call's final states, then decode steps: against one oracle run."""
    import torch

    T, H, d = 1500, 4, 128
    scale = 1.0 / np.sqrt(d)
    q, k, v = (la_inputs.normal(231, i, (T, H, d), "bf16", scale) for i in range(3))
    lam = np.array([0.9, 0.99, 0.5, 1.0], dtype=np.float32)
    cuts = [0, 333, 1000, 1490]
    state = None
    outs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, state = run(q[a:b], k[a:b], v[a:b], [0, b - a], 64, lam, state)
        outs.append(o)
    o_ref, kv_ref = oracle.recurrent(q, k, v, np.array([0, T], np.int32), decay=lam.astype(np.float64))
    ErrAcc().add(np.concatenate(outs), o_ref[:cuts[-1]]).check(False, "chunked decayed prefill o")
    # the last 10 tokens as decode steps (one sequence, H heads)
    S = to_dev(state)
    dl = to_dev(lam)
    for t in range(cuts[-1], T):
        od = la.decode(to_dev(q[t:t + 1]), to_dev(k[t:t + 1]), to_dev(v[t:t + 1]), S, decay=dl)
        torch.cuda.synchronize()
        ErrAcc().add(to_host(od)[0], o_ref[t]).check(False, f"decayed decode step {t}")
    ErrAcc().add(to_host(S)[0], kv_ref[0]).check(False, "decayed decode final state")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [32, 128])
def test_decay_decode_steps(dtype, d):
    """Decode steps on 64 (sequence, head) pairs of random states, per-head
    factors: every step's output and the final state against the oracle;
    lambda = 1 equal bit for bit to la_decode."""
    import torch

    ns, H = 16, 4
    lam = np.array([0.0, 0.6, 0.95, 1.0], dtype=np.float32)
    S0 = np.ascontiguousarray(la_inputs.normal(241, 4, (ns, H, d, d), "fp32", 0.1), dtype=np.float32)
    S = to_dev(S0)
    S_ref = S0.astype(np.float64).reshape(ns * H, d, d).copy()
    lam_pairs = np.tile(lam.astype(np.float64), ns)
    for step in range(5):
        q, k, v = la_inputs.decode_step_inputs(242, step, ns, H, d, dtype)
        o = la.decode(to_dev(q), to_dev(k), to_dev(v), S, decay=to_dev(lam))
        torch.cuda.synchronize()
        o_ref = oracle.decode_step(q.reshape(-1, d), k.reshape(-1, d), v.reshape(-1, d), S_ref, decay=lam_pairs)
        ErrAcc().add(to_host(o).reshape(-1, d), o_ref).check(dtype == "fp32", f"decode step {step} o")
    ErrAcc().add(to_host(S).reshape(-1, d, d), S_ref).check(True, "decode final state")
    # lambda = 1: the plain step, bit for bit
    S1, S2 = to_dev(S0), to_dev(S0)
    q, k, v = (to_dev(x) for x in la_inputs.decode_step_inputs(243, 0, ns, H, d, dtype))
    o1 = la.decode(q, k, v, S1, decay=to_dev(np.ones(H, np.float32)))
    o2 = la.decode(q, k, v, S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_decay_long_1m():
    """The 1M-token x 8-head workload with the decayed variant, compared in
    full with the oracle: per-head factors from 0.969 to 0.9998 (lambda_h =
    1 - 2^-(5+h)), so the scaled state is renormalised every few blocks on
    some heads and never on others, over 512-block segments with the
    segment states faded across the look-back and the scan."""
    import torch

    w = la_inputs.prefill_inputs("long_1m")
    T, H, d = w["T"], w["H"], w["d"]
    lam = np.array([1.0 - 2.0 ** -(5 + h) for h in range(H)], dtype=np.float32)
    plan = la.la_prefill_plan(T, 1, H, d, 64, la.LA_BF16)
    log(f"  decay long_1m plan={plan}")
    o, kv = run(w["q"], w["k"], w["v"], w["cu"], 64, lam)
    torch.cuda.empty_cache()
    acc_o, acc_kv = ErrAcc(), ErrAcc()
    for h0 in range(0, H, 4):
        o_ref, kv_ref = oracle.recurrent(w["q"], w["k"], w["v"], w["cu"], heads=(h0, h0 + 4),
                                         decay=lam.astype(np.float64))
        acc_o.add(o[:, h0:h0 + 4], o_ref)
        acc_kv.add(kv[:, h0:h0 + 4], kv_ref[:, h0:h0 + 4])
        log(f"    heads {h0}..{h0 + 3} compared")
        del o_ref
    acc_o.check(False, "decayed long_1m o")
    acc_kv.check(False, "decayed long_1m kv_state")

