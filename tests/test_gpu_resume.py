"""GPU parity of la_prefill_resume (prefill from given incoming states) and of
prefill and decode running concurrently on two streams.

Cases: random incoming states per document against the fp64 oracle (which
takes the same states), on every block loop, with segment splitting and the
scan path, with empty documents (whose final state is their incoming state);
a sequence prefilled in chunks, each chunk resuming from the previous chunk's
final state, against the single-call oracle result; and a mixed batch -- a
packed prefill on one stream and decode steps of other sequences on a second
stream at the same time -- against the oracle."""
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


def rand_inputs(seed, T, H, d, dtype):
    scale = 1.0 / np.sqrt(d)
    return [la_inputs.normal(seed, i, (T, H, d), dtype, scale) for i in range(3)]


def rand_states(seed, D, H, d, n_typical=2000):
    """fp32 states of the size a prefix of about n_typical tokens leaves
    (entries ~ N(0, n/d^2))."""
    s = la_inputs.normal(seed, 7, (D, H, d, d), "fp32", float(np.sqrt(n_typical)) / d)
    return np.ascontiguousarray(s, dtype=np.float32)


def run_resume(q, k, v, cu, kv_in, block, **opts):
    import torch

    o, kv = la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(np.asarray(cu, np.int32)), block=block,
                       kv_state_in=to_dev(kv_in), **opts)
    torch.cuda.synchronize()
    return to_host(o), to_host(kv)


CASES = [(d, block, dtype, opts)
         for d, block, dtype in ((128, 64, "bf16"), (64, 64, "bf16"), (128, 32, "bf16"), (32, 64, "fp32"))
         for opts in (dict(), dict(seg_len=2 * block, value_slices=2), dict(seg_len=block, force_scan=True))]


@pytest.mark.parametrize("d,block,dtype,opts", CASES, ids=[f"d{c[0]}-b{c[1]}-{c[2]}-{c[3]}" for c in CASES])
def test_resume_against_oracle(d, block, dtype, opts):
    lens = [300, 0, 1, 700, 64, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H = int(cu[-1]), 3
    q, k, v = rand_inputs(71 + d, T, H, d, dtype)
    kv_in = rand_states(72 + d, len(lens), H, d)
    log(f"  resume d={d} block={block} {dtype} {opts}")
    o, kv = run_resume(q, k, v, cu, kv_in, block, **opts)
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu, kv_in=kv_in)
    fp32 = dtype == "fp32"
    ErrAcc().add(o, o_ref).check(fp32, "resume o")
    ErrAcc().add(kv, kv_ref).check(fp32, "resume kv_state")
    for i, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(kv[i], kv_in[i]), "an empty document keeps its incoming state"


def test_resume_with_zero_states_is_prefill():
    """kv_state_in = 0 gives la_prefill's result bit for bit."""
    import torch

    T, H, d = 1000, 2, 128
    q, k, v = rand_inputs(81, T, H, d, "bf16")
    cu = np.array([0, 400, 1000], np.int32)
    o0, kv0 = la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(cu), block=64)
    o1, kv1 = la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(cu), block=64,
                         kv_state_in=torch.zeros((2, H, d, d), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(o0), to_host(o1)) and np.array_equal(to_host(kv0), to_host(kv1))


@pytest.mark.parametrize("chunk", [64, 1000, 4096])
def test_chunked_prefill(chunk):
    """A 12288-token sequence prefilled in chunks, each resuming from the
    state the previous chunk left, matches the oracle's single pass."""
    import torch

    T, H, d = 12288, 4, 128
    q, k, v = rand_inputs(91, T, H, d, "bf16")
    o_ref, kv_ref = oracle.recurrent(q, k, v, np.array([0, T], np.int32))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    state = torch.zeros((1, H, d, d), dtype=torch.float32, device="cuda")
    outs = []
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        o, state = la.prefill(qd[a:b], kd[a:b], vd[a:b], torch.tensor([0, b - a], dtype=torch.int32, device="cuda"),
                              block=64, kv_state_in=state)
        outs.append(o)
    torch.cuda.synchronize()
    log(f"  chunked prefill chunk={chunk}: {len(outs)} calls")
    ErrAcc().add(to_host(torch.cat(outs)), o_ref).check(False, f"chunked {chunk} o")
    ErrAcc().add(to_host(state), kv_ref).check(False, f"chunked {chunk} kv_state")


def test_prefill_and_decode_on_two_streams():
    """A packed prefill on one stream and 8 decode steps of an independent
    batch on another, launched back to back so they overlap, each checked
    against the oracle; then the same work serially gives identical bits."""
    import torch

    H, d = 8, 128
    lens = [1500, 3000, 700]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = rand_inputs(101, T, H, d, "bf16")
    ns = 64
    S0 = la_inputs.decode_states(105, ns, H, d, 2 * d, 1 << 16).reshape(ns, H, d, d)
    steps = [la_inputs.decode_step_inputs(106, s, ns, H, d, "bf16") for s in range(8)]

    def launch(sp, sd):
        qd, kd, vd, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(cu)
        S = torch.from_numpy(np.ascontiguousarray(S0)).cuda()
        dev_steps = [tuple(to_dev(x) for x in st) for st in steps]
        torch.cuda.synchronize()
        with torch.cuda.stream(sp):
            o_p, kv_p = la.prefill(qd, kd, vd, cud, block=64)
        with torch.cuda.stream(sd):
            o_d = [la.decode(*st, S) for st in dev_steps]
        torch.cuda.synchronize()
        return to_host(o_p), to_host(kv_p), [to_host(x) for x in o_d], to_host(S)

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o_p, kv_p, o_d, S = launch(s1, s2)
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu)
    ErrAcc().add(o_p, o_ref).check(False, "two-stream prefill o")
    ErrAcc().add(kv_p, kv_ref).check(False, "two-stream prefill kv_state")
    Sref = S0.astype(np.float64).reshape(ns * H, d, d).copy()
    acc = ErrAcc()
    for st, od in zip(steps, o_d):
        o_s = oracle.decode_step(*(x.reshape(-1, d) for x in st), Sref)
        acc.add(od.reshape(-1, d), o_s)
    acc.check(False, "two-stream decode o")
    ErrAcc().add(S.reshape(-1, d, d), Sref).check(True, "two-stream decode state")
    serial = torch.cuda.current_stream()
    o_p2, kv_p2, o_d2, S2 = launch(serial, serial)
    assert np.array_equal(o_p, o_p2) and np.array_equal(kv_p, kv_p2) and np.array_equal(S, S2)
    assert all(np.array_equal(a, b) for a, b in zip(o_d, o_d2))
