"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself: hand-worked examples
(tests/golden/hand_worked_d2.txt, and hand_worked_d2_decay.txt for the decayed
variant), closed forms that reduce to numpy or scipy routines (cumsum, tril,
matmul, a first-order recursive filter) or to a geometric series, algebraic identities of the definition (left product
== right product, split-then-resume, linearity, packed == separate), and the
two forms against each other.  ``test_planted_mistakes`` rebuilds the oracle
with one plausible mistake at a time and checks that some pin fails.

Definition followed: "MiniMax-01技术报告解读（一）模型架构" / "MiniMax-01技术报告解读",
§2.2 线性注意力 (right product, recursive key-value product, no softmax);
packed documents are independent (§3.2 items 1 and 4); decode is a length-1
step on the prefix key-value cache (§3.3 items 1-2).
"""
import os
import re

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_d2.txt")
TOL = 1e-12


def _close(a, b, tol=TOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    return a.shape == b.shape and (a.size == 0 or float(np.max(np.abs(a - b))) <= tol * scale)


def _rand(rng, T, H, d, dtype=np.float64):
    return [rng.standard_normal((T, H, d)).astype(dtype) for _ in range(3)]


def _golden():
    rows = {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, *vals = line.split()
            rows[name] = [float(x) for x in vals]
    return rows


# ----------------------------------------------------------------- pins

def pin_hand_worked(lib):
    g = _golden()
    toks = [g[f"tok{i}"] for i in range(1, 7)]
    q = np.array([t[0:2] for t in toks]).reshape(6, 1, 2)
    k = np.array([t[2:4] for t in toks]).reshape(6, 1, 2)
    v = np.array([t[4:6] for t in toks]).reshape(6, 1, 2)
    # documents: A = tokens 1..3, B = tokens 5..6 (token 4 is A's decode step)
    qa, ka, va = q[[0, 1, 2, 4, 5]], k[[0, 1, 2, 4, 5]], v[[0, 1, 2, 4, 5]]
    cu = np.array([0, 3, 5], dtype=np.int32)
    exp_o = np.array([g["o1"], g["o2"], g["o3"], g["o5"], g["o6"]]).reshape(5, 1, 2)
    exp_S = np.stack([np.array(g["S3"]).reshape(2, 2), np.array(g["S6"]).reshape(2, 2)]).reshape(2, 1, 2, 2)
    o_b, s_b = oracle.recurrent(qa, ka, va, cu, lib=lib)
    o_a, s_a = oracle.quadratic(qa, ka, va, cu, lib=lib)
    ok = np.array_equal(o_b, exp_o) and np.array_equal(s_b, exp_S)
    ok &= np.array_equal(o_a, exp_o) and np.array_equal(s_a, exp_S)
    # decode step of document A from S3
    S = np.array(g["S3"]).reshape(1, 2, 2).copy()
    o4 = oracle.decode_step(q[3].reshape(1, 2), k[3].reshape(1, 2), v[3].reshape(1, 2), S, lib=lib)
    ok &= np.array_equal(o4, np.array([g["o4"]])) and np.array_equal(S.reshape(4), np.array(g["S4"]))
    return bool(ok)


def pin_forms_agree(lib, seeds=range(4)):
    for seed in seeds:
        rng = np.random.default_rng(1000 + seed)
        for n in (1, 2, 3, 7, 64):
            for d in (1, 2, 16):
                for H in (1, 2):
                    q, k, v = _rand(rng, n, H, d)
                    cu = np.array([0, n], dtype=np.int32)
                    kv_in = rng.standard_normal((1, H, d, d)) if (seed % 2) else None
                    ob, sb = oracle.recurrent(q, k, v, cu, kv_in=kv_in, lib=lib)
                    oa, sa = oracle.quadratic(q, k, v, cu, kv_in=kv_in, lib=lib)
                    if not (_close(ob, oa) and _close(sb, sa)):
                        return False
    # varlen with empty documents
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 40, 2, 5)
    cu = np.array([0, 0, 9, 9, 30, 40, 40], dtype=np.int32)
    ob, sb = oracle.recurrent(q, k, v, cu, lib=lib)
    oa, sa = oracle.quadratic(q, k, v, cu, lib=lib)
    return _close(ob, oa) and _close(sb, sa)


def pin_split_resume(lib):
    rng = np.random.default_rng(11)
    n, H, d = 24, 2, 6
    q, k, v = _rand(rng, n, H, d)
    o_full, s_full = oracle.recurrent(q, k, v, np.array([0, n], np.int32), lib=lib)
    for m in range(0, n + 1):
        _, s_m = oracle.recurrent(q[:m], k[:m], v[:m], np.array([0, m], np.int32), want_o=False, lib=lib)
        o_t, s_t = oracle.recurrent(q[m:], k[m:], v[m:], np.array([0, n - m], np.int32), kv_in=s_m, lib=lib)
        if not (_close(o_t, o_full[m:]) and _close(s_t, s_full)):
            return False
    return True


def pin_closed_forms(lib):
    rng = np.random.default_rng(5)
    # n = 1: o = (q . k) v
    q, k, v = _rand(rng, 1, 3, 8)
    o, s = oracle.recurrent(q, k, v, np.array([0, 1], np.int32), lib=lib)
    if not _close(o[0], np.einsum("hi,hi->h", q[0], k[0])[:, None] * v[0]):
        return False
    if not _close(s[0], np.einsum("hi,hj->hij", k[0], v[0])):
        return False
    # d = 1: O_t = q_t * cumsum(k_s v_s)
    q, k, v = _rand(rng, 50, 1, 1)
    o, _ = oracle.recurrent(q, k, v, np.array([0, 50], np.int32), lib=lib)
    if not _close(o[:, 0, 0], q[:, 0, 0] * np.cumsum(k[:, 0, 0] * v[:, 0, 0])):
        return False
    # q_t = k_s = e_1: O_t = cumsum(v)
    n, d = 33, 4
    e1 = np.zeros((n, 1, d))
    e1[:, 0, 0] = 1.0
    v = rng.standard_normal((n, 1, d))
    o, _ = oracle.recurrent(e1, e1.copy(), v, np.array([0, n], np.int32), lib=lib)
    if not _close(o[:, 0, :], np.cumsum(v[:, 0, :], axis=0)):
        return False
    # V = I (n = d): O = tril(Q K^T) -- pins mask orientation and the diagonal
    n = d = 9
    q = rng.standard_normal((n, 1, d))
    k = rng.standard_normal((n, 1, d))
    eye = np.eye(n).reshape(n, 1, d)
    for fn in (oracle.recurrent, oracle.quadratic):
        o, _ = fn(q, k, eye, np.array([0, n], np.int32), lib=lib)
        if not _close(o[:, 0, :], np.tril(q[:, 0, :] @ k[:, 0, :].T)):
            return False
    # kv_out = K^T V via numpy matmul
    q, k, v = _rand(rng, 70, 2, 7)
    _, s = oracle.recurrent(q, k, v, np.array([0, 70], np.int32), want_o=False, lib=lib)
    for h in range(2):
        if not _close(s[0, h], k[:, h, :].T @ v[:, h, :]):
            return False
    return True


def pin_linearity(lib):
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 30, 2, 5)
    v2 = rng.standard_normal(v.shape)
    q2 = rng.standard_normal(q.shape)
    cu = np.array([0, 30], np.int32)
    a, b = 1.75, -0.5
    o1, _ = oracle.recurrent(q, k, v, cu, lib=lib)
    o2, _ = oracle.recurrent(q, k, v2, cu, lib=lib)
    o3, _ = oracle.recurrent(q, k, a * v + b * v2, cu, lib=lib)
    if not _close(o3, a * o1 + b * o2, 1e-11):
        return False
    o4, _ = oracle.recurrent(q2, k, v, cu, lib=lib)
    o5, _ = oracle.recurrent(a * q + b * q2, k, v, cu, lib=lib)
    return _close(o5, a * o1 + b * o4, 1e-11)


def pin_packed_equals_separate(lib):
    rng = np.random.default_rng(13)
    lens = [5, 0, 17, 1, 0, 9]
    T = sum(lens)
    q, k, v = _rand(rng, T, 3, 4)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, s = oracle.recurrent(q, k, v, cu, lib=lib)
    for i, n in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        oi, si = oracle.recurrent(q[a:b], k[a:b], v[a:b], np.array([0, n], np.int32), lib=lib)
        if not (_close(o[a:b], oi) and _close(s[i], si[0])):
            return False
        if n == 0 and np.any(s[i] != 0):
            return False
    return True


def pin_decode_continues_prefill(lib):
    rng = np.random.default_rng(17)
    n, H, d = 12, 2, 8
    q, k, v = _rand(rng, n, H, d)
    o_full, s_full = oracle.recurrent(q, k, v, np.array([0, n], np.int32), lib=lib)
    m = 7
    _, S = oracle.recurrent(q[:m], k[:m], v[:m], np.array([0, m], np.int32), want_o=False, lib=lib)
    S = S[0].copy()
    for t in range(m, n):
        o_t = oracle.decode_step(q[t], k[t], v[t], S, lib=lib)
        if not _close(o_t, o_full[t]):
            return False
    # closed form of one step: S' = S + k^T v, o = q . S'
    S0 = rng.standard_normal((3, d, d))
    qq, kk, vv = (rng.standard_normal((3, d)) for _ in range(3))
    S1 = S0.copy()
    o = oracle.decode_step(qq, kk, vv, S1, lib=lib)
    ref_S = S0 + np.einsum("pi,pj->pij", kk, vv)
    return _close(S1, ref_S) and _close(o, np.einsum("pi,pij->pj", qq, ref_S))


def pin_backward_finite_differences(lib):
    """The backward against central differences of the forward.  The loss
    L = sum(dO * o) + sum(dKV_out * kv_out) is affine in any single input
    element (o is linear in each of q, k, v and kv_in), so a central
    difference with step 1 equals the derivative up to rounding."""
    rng = np.random.default_rng(31)
    T, H, d = 9, 2, 3
    cu = np.array([0, 4, 4, 9], np.int32)
    q, k, v, dout = (rng.standard_normal((T, H, d)) for _ in range(4))
    kv_in, dkv_out = (rng.standard_normal((3, H, d, d)) for _ in range(2))

    def loss(q_, k_, v_, kv_):
        o, kvo = oracle.recurrent(q_, k_, v_, cu, kv_in=kv_, nthreads=1, lib=lib)
        return float(np.sum(dout * o) + np.sum(dkv_out * kvo))

    grads = oracle.backward(q, k, v, dout, cu, kv_in=kv_in, dkv_out=dkv_out, nthreads=1, lib=lib)
    args = [q, k, v, kv_in]
    for which, g in enumerate((grads[0], grads[1], grads[2], grads[3])):
        fd = np.empty_like(args[which])
        for idx in np.ndindex(args[which].shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += 1.0
            minus[which][idx] -= 1.0
            fd[idx] = 0.5 * (loss(*plus) - loss(*minus))
        if not _close(g, fd, 1e-10):
            return False
    return True


# ------------------------------------------------------ decayed variant

GOLDEN_DECAY = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_d2_decay.txt")


def pin_decay_hand_worked(lib):
    g = {}
    with open(GOLDEN_DECAY, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                name, *vals = line.split()
                g[name] = [float(x) for x in vals]
    lam = np.array(g["lambda"])
    toks = [g[f"tok{i}"] for i in range(1, 7)]
    q = np.array([t[0:2] for t in toks]).reshape(6, 1, 2)
    k = np.array([t[2:4] for t in toks]).reshape(6, 1, 2)
    v = np.array([t[4:6] for t in toks]).reshape(6, 1, 2)
    sel = [0, 1, 2, 4, 5]
    cu = np.array([0, 3, 5], dtype=np.int32)
    exp_o = np.array([g["o1"], g["o2"], g["o3"], g["o5"], g["o6"]]).reshape(5, 1, 2)
    exp_S = np.stack([np.array(g["S3"]).reshape(2, 2), np.array(g["S6"]).reshape(2, 2)]).reshape(2, 1, 2, 2)
    ok = True
    for fn in (oracle.recurrent, oracle.quadratic):
        o, s = fn(q[sel], k[sel], v[sel], cu, lib=lib, decay=lam)
        ok &= np.array_equal(o, exp_o) and np.array_equal(s, exp_S)
    S = np.array(g["S3"]).reshape(1, 2, 2).copy()
    o4 = oracle.decode_step(q[3].reshape(1, 2), k[3].reshape(1, 2), v[3].reshape(1, 2), S, lib=lib, decay=lam)
    ok &= np.array_equal(o4, np.array([g["o4"]])) and np.array_equal(S.reshape(4), np.array(g["S4"]))
    return bool(ok)


def pin_decay_one_is_undecayed(lib):
    """lambda = 1 gives the undecayed results bit for bit (every form)."""
    rng = np.random.default_rng(41)
    q, k, v = _rand(rng, 37, 3, 6)
    cu = np.array([0, 10, 10, 37], np.int32)
    kv_in = rng.standard_normal((3, 3, 6, 6))
    ones = np.ones(3)
    for fn in (oracle.recurrent, oracle.quadratic):
        a = fn(q, k, v, cu, kv_in=kv_in, lib=lib)
        b = fn(q, k, v, cu, kv_in=kv_in, lib=lib, decay=ones)
        if not (np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])):
            return False
    S0 = rng.standard_normal((4, 6, 6))
    qq, kk, vv = (rng.standard_normal((4, 6)) for _ in range(3))
    S1, S2 = S0.copy(), S0.copy()
    o1 = oracle.decode_step(qq, kk, vv, S1, lib=lib)
    o2 = oracle.decode_step(qq, kk, vv, S2, lib=lib, decay=np.ones(4))
    return np.array_equal(o1, o2) and np.array_equal(S1, S2)


def pin_decay_forms_agree(lib):
    """Recurrent and quadratic decayed forms, per-head factors including 0 and
    1, with and without incoming states, packed documents with empty ones."""
    rng = np.random.default_rng(43)
    for lam in ([0.0, 0.25, 0.9, 1.0], [0.5, 0.5, 0.5, 0.5], [0.999, 0.1, 0.0, 0.7]):
        for kv in (False, True):
            q, k, v = _rand(rng, 45, 4, 5)
            cu = np.array([0, 0, 13, 13, 40, 45], np.int32)
            kv_in = rng.standard_normal((5, 4, 5, 5)) if kv else None
            ob, sb = oracle.recurrent(q, k, v, cu, kv_in=kv_in, lib=lib, decay=lam)
            oa, sa = oracle.quadratic(q, k, v, cu, kv_in=kv_in, lib=lib, decay=lam)
            if not (_close(ob, oa) and _close(sb, sa)):
                return False
    return True


def pin_decay_closed_forms(lib):
    from scipy.signal import lfilter

    rng = np.random.default_rng(47)
    # d = 1: the state is the first-order recursive filter y_t = x_t + lambda y_{t-1}
    # of x_t = k_t v_t (scipy's lfilter), and o_t = q_t y_t
    n, lam = 80, 0.83
    q, k, v = _rand(rng, n, 1, 1)
    o, s = oracle.recurrent(q, k, v, np.array([0, n], np.int32), lib=lib, decay=[lam])
    y = lfilter([1.0], [1.0, -lam], k[:, 0, 0] * v[:, 0, 0])
    if not (_close(o[:, 0, 0], q[:, 0, 0] * y) and _close(s[0, 0, 0, 0], y[-1])):
        return False
    # q_t = k_t = e_1, v_t = u: a geometric series, o_t = u (1 - lambda^(t+1)) / (1 - lambda)
    n, d, lam = 30, 3, 0.6
    e1 = np.zeros((n, 1, d))
    e1[:, 0, 0] = 1.0
    u = rng.standard_normal(d)
    vv = np.tile(u, (n, 1)).reshape(n, 1, d)
    o, _ = oracle.recurrent(e1, e1.copy(), vv, np.array([0, n], np.int32), lib=lib, decay=[lam])
    t = np.arange(n)[:, None]
    if not _close(o[:, 0, :], u[None, :] * (1.0 - lam ** (t + 1)) / (1.0 - lam)):
        return False
    # lambda = 0: only the current token (and no incoming state) survives: o_t = (q_t . k_t) v_t
    q, k, v = _rand(rng, 20, 2, 4)
    kv_in = rng.standard_normal((1, 2, 4, 4))
    o, s = oracle.recurrent(q, k, v, np.array([0, 20], np.int32), kv_in=kv_in, lib=lib, decay=[0.0, 0.0])
    if not _close(o, np.einsum("thi,thi->th", q, k)[:, :, None] * v):
        return False
    if not _close(s[0], np.einsum("hi,hj->hij", k[-1], v[-1])):
        return False
    # per-head factors: each head equals a one-head run with its own factor
    q, k, v = _rand(rng, 25, 3, 4)
    lams = [0.2, 0.95, 0.6]
    cu = np.array([0, 25], np.int32)
    o, s = oracle.recurrent(q, k, v, cu, lib=lib, decay=lams)
    for h in range(3):
        oh, sh = oracle.recurrent(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], cu, lib=lib, decay=[lams[h]])
        if not (_close(o[:, h:h + 1], oh) and _close(s[:, h:h + 1], sh)):
            return False
    return True


def pin_decay_split_resume(lib):
    rng = np.random.default_rng(53)
    n, H, d = 20, 2, 5
    lam = [0.7, 0.95]
    q, k, v = _rand(rng, n, H, d)
    o_full, s_full = oracle.recurrent(q, k, v, np.array([0, n], np.int32), lib=lib, decay=lam)
    for m in range(0, n + 1):
        _, s_m = oracle.recurrent(q[:m], k[:m], v[:m], np.array([0, m], np.int32), want_o=False, lib=lib, decay=lam)
        o_t, s_t = oracle.recurrent(q[m:], k[m:], v[m:], np.array([0, n - m], np.int32), kv_in=s_m, lib=lib,
                                    decay=lam)
        if not (_close(o_t, o_full[m:]) and _close(s_t, s_full)):
            return False
    # decode continues the decayed prefill
    m = 12
    _, S = oracle.recurrent(q[:m], k[:m], v[:m], np.array([0, m], np.int32), want_o=False, lib=lib, decay=lam)
    S = S[0].copy()
    for t in range(m, n):
        if not _close(oracle.decode_step(q[t], k[t], v[t], S, lib=lib, decay=lam), o_full[t]):
            return False
    return True


PINS = [pin_hand_worked, pin_forms_agree, pin_split_resume, pin_closed_forms, pin_linearity,
        pin_packed_equals_separate, pin_decode_continues_prefill, pin_backward_finite_differences,
        pin_decay_hand_worked, pin_decay_one_is_undecayed, pin_decay_forms_agree, pin_decay_closed_forms,
        pin_decay_split_resume]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(oracle_lib, pin):
    assert pin(oracle_lib)


def test_dtype_widening_is_exact(oracle_lib):
    """bf16 bit patterns and fp32 inputs give the same fp64 result as their exact values."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 2, 8)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: exactly representable values
    xb = (bits.astype(np.uint32) << 16).view(np.float32)
    cu = np.array([0, 20], np.int32)
    o16, s16 = oracle.recurrent(bits, bits, bits, cu)
    o64, s64 = oracle.recurrent(xb.astype(np.float64), xb.astype(np.float64), xb.astype(np.float64), cu)
    assert np.array_equal(o16, o64) and np.array_equal(s16, s64)
    o32, _ = oracle.recurrent(x, x, x, cu)
    o64b, _ = oracle.recurrent(x.astype(np.float64), x.astype(np.float64), x.astype(np.float64), cu)
    assert np.array_equal(o32, o64b)


def test_thread_count_invariance(oracle_lib):
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 200, 3, 40)
    cu = np.array([0, 50, 120, 200], np.int32)
    a = oracle.recurrent(q, k, v, cu, nthreads=1)
    b = oracle.recurrent(q, k, v, cu, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_head_range(oracle_lib):
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 30, 4, 6)
    cu = np.array([0, 30], np.int32)
    o, s = oracle.recurrent(q, k, v, cu)
    o2, s2 = oracle.recurrent(q, k, v, cu, heads=(1, 3))
    assert np.array_equal(o2, o[:, 1:3]) and np.array_equal(s2[:, 1:3], s[:, 1:3])


# ------------------------------------------------------- planted mistakes

# (description, regex in la_oracle.c, replacement).  Each is a plausible slip
# when writing the method; each must make at least one pin fail.
MUTANTS = [
    ("recurrent: k replaced by q in the state update",
     r"kk\[i\] \* vv\[jj\]", "qq[i] * vv[jj]"),
    ("recurrent: state sign flipped",
     r"S\[i \* ORA_COLS \+ jj\] \+= kk\[i\] \* vv\[jj\]", "S[i * ORA_COLS + jj] -= kk[i] * vv[jj]"),
    ("recurrent: k and v swapped (transposed state)",
     r"kk\[i\] = widen\(c->k,", "kk[i] = widen(c->v,"),
    ("recurrent: no reset at document start",
     r"for \(int64_t t = c->cu\[doc\];", "for (int64_t t = 0;"),
    ("recurrent: output read from the wrong row of the state",
     r"acc\[jj\] \+= qq\[i\] \* S\[i \* ORA_COLS \+ jj\]", "acc[jj] += qq[i] * S[((i + 1) % d) * ORA_COLS + jj]"),
    ("quadratic: diagonal dropped from the causal mask",
     r"for \(int64_t cc = 0; cc <= r; \+\+cc\)", "for (int64_t cc = 0; cc < r; ++cc)"),
    ("quadratic: kv_in term dropped",
     r"if \(kv_in\)\n(\s+)for \(int32_t i = 0; i < d; \+\+i\) acc \+= widen\(q",
     "if (0)\n\\1for (int32_t i = 0; i < d; ++i) acc += widen(q"),
    ("decode: k and v swapped",
     r"double ki = widen\(c->k,", "double ki = widen(c->v,"),
    ("decode: output read before the update",
     r"/\* S <- S \+ k\^T v \*/\n(\s+)for \(int32_t i = 0; i < d; \+\+i\) \{\n(\s+)double ki",
     "/* S <- S + k^T v */\n\\1if (c->o) for (int32_t j = 0; j < d; ++j) { double a0 = 0.0; for (int32_t i = 0; i < d; ++i) a0 += widen(c->q, c->dtype, row + i) * S[(size_t)i * d + j]; c->o[row + j] = a0; }\n\\1if (c->o) return;\n\\1for (int32_t i = 0; i < d; ++i) {\n\\2double ki"),
    ("backward: dKV_out ignored",
     r"M\[e\] = c->dkv_out \? c->dkv_out\[sbase \+ e\] : 0\.0;", "M[e] = 0.0;"),
    ("backward: dq from the transposed state",
     r"acc \+= M\[\(size_t\)i \* d \+ j\] \* b\[j\];\n(\s+)c->dq", "acc += M[(size_t)j * d + i] * b[j];\n\\1c->dq"),
    ("backward: dv from the transposed reverse state",
     r"acc \+= a\[i\] \* M\[\(size_t\)i \* d \+ j\];", "acc += a[i] * M[(size_t)j * d + i];"),
    ("decay: factor ignored in the recurrence",
     r"S\[i \* ORA_COLS \+ jj\] \*= c->decay\[h\];", "S[i * ORA_COLS + jj] *= 1.0;"),
    ("decay: the first head's factor for every head",
     r"S\[i \* ORA_COLS \+ jj\] \*= c->decay\[h\];", "S[i * ORA_COLS + jj] *= c->decay[0];"),
    ("decay: quadratic form's exponent off by one",
     r"pow\(lam, \(double\)\(r - cc\)\)", "pow(lam, (double)(r - cc + 1))"),
    ("decay: incoming state not faded in the quadratic form",
     r"const double f = pow\(lam, \(double\)\(r \+ 1\)\);", "const double f = 1.0;"),
    ("decay: decode fades the state twice",
     r"S\[e\] \*= c->decay\[p\];", "S[e] *= c->decay[p] * c->decay[p];"),
    ("backward: token s left out of its own reverse sum",
     r"(\s+)for \(int32_t i = 0; i < d; \+\+i\) a\[i\] = widen\(c->q, c->dtype, row \+ i\);",
     "\\1for (int32_t i = 0; i < d; ++i) a[i] = (t == (int64_t)c->cu[doc + 1] - 1) ? 0.0 : widen(c->q, c->dtype, row + i + H * d);"),
]


@pytest.mark.parametrize("desc,pat,rep", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes(tmp_path, oracle_lib, desc, pat, rep):
    src = open(oracle._SRC, encoding="utf-8").read()
    mutated, n = re.subn(pat, rep, src, count=1)
    assert n == 1, f"mutation pattern not found: {desc}"
    msrc = tmp_path / "la_oracle.c"
    msrc.write_text(mutated, encoding="utf-8")
    import shutil
    import subprocess

    shutil.copy(os.path.join(os.path.dirname(oracle._SRC), "la_oracle.h"), tmp_path / "la_oracle.h")
    so = str(tmp_path / "mut.so")
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", str(msrc), "-o", so, "-lm"])
    lib = oracle.load(so)
    failed = []
    for pin in PINS:
        try:
            ok = pin(lib)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake: {desc}"
