"""GPU parity of la_decode against the fp64 oracle (through the C ABI).

Cases: every d and dtype over several steps; prefill followed by decode
equals a longer prefill; and the 256-sequence x 64-head workload with its
sampled incoming states over 1000 consecutive steps (outputs of sampled pairs
at every step, all pairs at the last step, and the final state of every pair
against the closed form S_0 + sum of k^T v)."""
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


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_decode_steps(d, dtype):
    import torch

    ns, H, steps = 5, 3, 6
    S0 = la_inputs.decode_states(11 + d, ns, H, d, 2 * d, 4096)
    S_gpu = to_dev(S0.reshape(ns, H, d, d).copy())
    S_ref = S0.astype(np.float64).reshape(ns * H, d, d).copy()
    acc_o = ErrAcc()
    for s in range(steps):
        q, k, v = la_inputs.decode_step_inputs(19 + d, s, ns, H, d, dtype)
        log(f"  decode d={d} {dtype} step {s}")
        o = la.decode(to_dev(q), to_dev(k), to_dev(v), S_gpu)
        torch.cuda.synchronize()
        o_ref = oracle.decode_step(q.reshape(-1, d), k.reshape(-1, d), v.reshape(-1, d), S_ref)
        acc_o.add(to_host(o).reshape(-1, d), o_ref)
    acc_o.check(dtype == "fp32", f"decode d={d} {dtype} o")
    ErrAcc().add(to_host(S_gpu).reshape(-1, d, d), S_ref).check(True, f"decode d={d} {dtype} state")


def test_prefill_then_decode_continues():
    """prefill(n - m) followed by m decode steps gives the outputs of prefill(n)."""
    import torch

    T, H, d, m = 300, 4, 128, 9
    scale = 1 / np.sqrt(d)
    q, k, v = (la_inputs.normal(23, i, (T, H, d), "bf16", scale) for i in range(3))
    o_full, kv_full = la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(np.array([0, T], np.int32)), block=64)
    n0 = T - m
    o_head, kv = la.prefill(to_dev(q[:n0]), to_dev(k[:n0]), to_dev(v[:n0]), to_dev(np.array([0, n0], np.int32)),
                            block=64)
    outs = []
    for t in range(n0, T):
        outs.append(to_host(la.decode(to_dev(q[t:t + 1]), to_dev(k[t:t + 1]), to_dev(v[t:t + 1]), kv)))
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.recurrent(q, k, v, np.array([0, T], np.int32))
    ErrAcc().add(np.concatenate(outs, 0), o_ref[n0:]).check(False, "decoded tail o")
    ErrAcc().add(to_host(kv), kv_ref).check(False, "state after decode")
    ErrAcc().add(to_host(o_full)[n0:], o_ref[n0:]).check(False, "prefill tail o")


def test_decode_workload_1000_steps():
    import torch

    cfg = la_inputs.WORKLOADS["decode_256x64"]
    ns, H, d, seed, steps, pool = cfg["num_seqs"], cfg["H"], cfg["d"], cfg["seed"], cfg["steps"], cfg["pool"]
    lo, hi = cfg["prefix"]
    P = ns * H
    log(f"  decode workload {ns}x{H} d={d} steps={steps} pool={pool}: sampling incoming states")
    S0 = la_inputs.decode_states(seed, ns, H, d, lo, hi)  # fp32 [P, d, d]
    S_gpu = to_dev(S0.reshape(ns, H, d, d))
    sets = [la_inputs.decode_step_inputs(seed, s, ns, H, d, "bf16") for s in range(pool)]
    dev_sets = [tuple(to_dev(x) for x in st) for st in sets]
    rng = np.random.default_rng(seed)
    sample = np.sort(rng.choice(P, size=512, replace=False))
    S_ref = S0.reshape(P, d, d)[sample].astype(np.float64)
    acc_o = ErrAcc()
    o_hist = []
    for s in range(steps):
        q, k, v = dev_sets[s % pool]
        o = la.decode(q, k, v, S_gpu)
        o_hist.append(o[:, :, :].reshape(P, d)[torch.from_numpy(sample).cuda()].clone())
        if s % 100 == 0:
            log(f"    step {s}")
    torch.cuda.synchronize()
    for s in range(steps):
        qh, kh, vh = (x.reshape(P, d)[sample] for x in sets[s % pool])
        o_ref = oracle.decode_step(qh, kh, vh, S_ref)
        acc_o.add(to_host(o_hist[s]), o_ref)
    acc_o.check(False, "sampled pairs, every step, o")
    # closed form for every pair: S_final = S_0 + sum_s count_s k_s^T v_s
    counts = np.bincount(np.arange(steps) % pool, minlength=pool).astype(np.float64)
    K_all = np.stack([as_f64(sets[s][1].reshape(P, d)) * counts[s] for s in range(pool)], axis=1)  # [P, pool, d]
    V_all = np.stack([as_f64(sets[s][2].reshape(P, d)) for s in range(pool)], axis=1)
    S_fin = S0.reshape(P, d, d).astype(np.float64) + np.matmul(K_all.transpose(0, 2, 1), V_all)
    del K_all, V_all
    S_last = to_host(S_gpu).reshape(P, d, d)
    ErrAcc().add(S_last, S_fin).check(True, "final state, all pairs")
    log(f"    final state rel_l2 {ErrAcc().add(S_last, S_fin).rel_l2:.3e}")
    q_last = as_f64(sets[(steps - 1) % pool][0].reshape(P, d))
    o_last_ref = np.einsum("pi,pij->pj", q_last, S_fin)
    ErrAcc().add(to_host(o).reshape(P, d), o_last_ref).check(False, "last step o, all pairs")
