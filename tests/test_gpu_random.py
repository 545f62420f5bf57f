"""Randomised parity: seeded draws of shapes, packed-document layouts and
every decomposition knob (segment length, value slices, scan, tile slots,
block loop, work list, incoming states), each prefill checked against the fp64 oracle,
and a share of them through the backward and the decayed prefill (per-head
factors drawn from 0, 1, (0.9, 1] and [0, 1)) as well.  Draws whose options the
planner rejects must be rejected (LA_ERR_UNSUPPORTED) before anything runs."""
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


def draw(seed):
    """One configuration from a counter-seeded generator (numpy's PCG64)."""
    r = np.random.default_rng(seed)
    d = int(r.choice([32, 64, 128]))
    dtype = "fp32" if r.random() < 0.2 else "bf16"
    block = int(r.choice([32, 64, 128] if dtype == "bf16" else [32, 64]))
    H = int(r.integers(1, 5))
    ndocs = int(r.integers(1, 7))
    lens = [int(x) for x in r.integers(0, 900, ndocs)]
    if r.random() < 0.3:
        lens[int(r.integers(0, ndocs))] = 0
    if sum(lens) == 0:
        lens[0] = int(r.integers(1, 500))
    opts = {}
    if r.random() < 0.6:
        opts["seg_len"] = block * int(r.integers(1, 12))
    if r.random() < 0.4:
        opts["value_slices"] = int(r.choice([1, 2, 4]))
    if r.random() < 0.3:
        opts["force_scan"] = True
    if r.random() < 0.3:
        opts["variant"] = int(r.choice([1, 2]))
    if r.random() < 0.3:
        opts["slots"] = int(r.choice([2, 3]))
    kv_in = r.random() < 0.4
    backward = r.random() < 0.35
    if r.random() < 0.35:  # drawn last: the earlier knobs of every seed stay as they were
        opts["work_list"] = int(r.choice([1, 2]))
    decay = None
    if r.random() < 0.3:  # (after the work list, for the same reason)
        kind = r.integers(0, 4, H)
        near_one, anywhere = 1.0 - 0.1 * r.random(H), r.random(H)
        lam = np.where(kind == 0, 1.0, np.where(kind == 1, 0.0, np.where(kind == 2, near_one, anywhere)))
        decay = [float(np.float32(x)) for x in lam]
    return dict(d=d, dtype=dtype, block=block, H=H, lens=lens, opts=opts, kv_in=kv_in, backward=backward, decay=decay)


SEEDS = list(range(1000, 2000))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(seed):
    import torch

    c = draw(seed)
    d, H, block, dtype, opts = c["d"], c["H"], c["block"], c["dtype"], c["opts"]
    cu = np.concatenate([[0], np.cumsum(c["lens"])]).astype(np.int32)
    T, D = int(cu[-1]), len(c["lens"])
    dt = la.LA_BF16 if dtype == "bf16" else la.LA_FP32
    try:
        plan = la.la_prefill_plan(T, D, H, d, block, dt, la.make_opts(**opts))
    except la.LAError as e:
        # a rejected combination is rejected by the call too, before anything is enqueued
        assert e.status == la.LA_ERR_UNSUPPORTED
        q = to_dev(la_inputs.normal(seed, 0, (T, H, d), dtype, 1.0))
        with pytest.raises(la.LAError):
            la.prefill(q, q, q, to_dev(cu), block=block, **opts)
        log(f"  seed {seed}: rejected {c}")
        return
    log(f"  seed {seed}: {c} plan={plan}")
    scale = 1.0 / np.sqrt(d)
    q, k, v = (la_inputs.normal(seed, i, (T, H, d), dtype, scale) for i in range(3))
    kv_in = None
    if c["kv_in"]:
        kv_in = np.ascontiguousarray(la_inputs.normal(seed, 7, (D, H, d, d), "fp32", float(np.sqrt(500)) / d),
                                     dtype=np.float32)
    qd, kd, vd, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(cu)
    kin = None if kv_in is None else to_dev(kv_in)
    o, kv = la.prefill(qd, kd, vd, cud, block=block, kv_state_in=kin, **opts)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu, kv_in=kv_in)
    fp32 = dtype == "fp32"
    ErrAcc().add(to_host(o), o_ref).check(fp32, f"seed {seed} o")
    ErrAcc().add(to_host(kv), kv_ref).check(fp32, f"seed {seed} kv_state")
    if c["backward"]:
        dout = la_inputs.normal(seed, 8, (T, H, d), dtype, 1.0)
        dko = np.ascontiguousarray(la_inputs.normal(seed, 9, (D, H, d, d), "fp32", 1.0), dtype=np.float32)
        got = la.backward(qd, kd, vd, to_dev(dout), cud, block=block, kv_state_in=kin, dkv_state_out=to_dev(dko),
                          **opts)
        torch.cuda.synchronize()
        ref = oracle.backward(q, k, v, dout, cu, kv_in=kv_in, dkv_out=dko)
        for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            ErrAcc().add(to_host(g), r).check(fp32, f"seed {seed} {name}")
        ErrAcc().add(to_host(got[3]), ref[3]).check(True, f"seed {seed} dkv_in")
    if c["decay"] is not None:
        lam = np.array(c["decay"], np.float32)
        try:
            od, kvd = la.prefill(qd, kd, vd, cud, block=block, kv_state_in=kin, decay=to_dev(lam), **opts)
        except la.LAError as e:
            # The decayed kernels differ from the plain ones only where they have no room:
            # no 128-token transpose-read loop (so options chosen for it may not fit the
            # generic one) and no third tile slot at full width (d = 128, one slice).
            assert e.status == la.LA_ERR_UNSUPPORTED
            at_b128 = block == 128 and any(x in opts for x in ("variant", "value_slices", "slots", "seg_len",
                                                                "work_list"))
            three_wide = opts.get("slots") == 3 and d == 128
            assert at_b128 or three_wide, f"seed {seed}: decayed call rejected {c}"
            log(f"  seed {seed}: decayed call rejected")
            return
        torch.cuda.synchronize()
        o_ref, kv_ref = oracle.recurrent(q, k, v, cu, kv_in=kv_in, decay=lam.astype(np.float64))
        ErrAcc().add(to_host(od), o_ref).check(fp32, f"seed {seed} decayed o")
        ErrAcc().add(to_host(kvd), kv_ref).check(fp32, f"seed {seed} decayed kv_state")
