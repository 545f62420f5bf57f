"""GPU parity of la_prefill against the fp64 oracle (through the C ABI).

Cases: the tiny fp32 and 8k-token bf16 workloads in full; every (d, block,
dtype) the library supports on ragged lengths; forced segment splitting and
value slicing (the LASP+-style prefix path); the document-piece work list
(documents cut into pieces, longest first, on every block loop); two and three tile slots in the
block loop; packed documents with empty and ragged ones; exact-integer
inputs that must match bit for bit; run-to-run
determinism; guard bands around the outputs; zero tokens; and the
131072-token varlen and 1M-token workloads in full, in the launch
configuration the benchmark uses."""
import ctypes

import numpy as np
import pytest

import causal_linear_attention_la_amd as la
import la_inputs
import oracle
from gpu_helpers import ErrAcc, as_f64, bf16_rne_from_f64, log, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    la.load()  # the HIP library must be present: no fallback
    la_inputs.build()
    oracle.build()
    yield


def run_gpu(q, k, v, cu, block, **opts):
    import torch

    qd, kd, vd, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(np.asarray(cu, dtype=np.int32))
    o, kv = la.prefill(qd, kd, vd, cud, block=block, **opts)
    torch.cuda.synchronize()
    return to_host(o), to_host(kv)


def check_against_oracle(q, k, v, cu, o_gpu, kv_gpu, fp32, what):
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu)
    ErrAcc().add(o_gpu, o_ref).check(fp32, f"{what} o")
    ErrAcc().add(kv_gpu, kv_ref).check(fp32, f"{what} kv_state")
    return o_ref, kv_ref


def rand_inputs(seed, T, H, d, dtype):
    scale = 1.0 / np.sqrt(d)
    return [la_inputs.normal(seed, i, (T, H, d), dtype, scale) for i in range(3)]


def test_tiny_fp32_workload():
    w = la_inputs.prefill_inputs("tiny_fp32")
    log(f"  tiny_fp32 T={w['T']} H={w['H']} d={w['d']} block={w['block']}")
    o, kv = run_gpu(w["q"], w["k"], w["v"], w["cu"], w["block"])
    check_against_oracle(w["q"], w["k"], w["v"], w["cu"], o, kv, True, "tiny_fp32")


def test_prefill_8k_workload():
    w = la_inputs.prefill_inputs("prefill_8k")
    log(f"  prefill_8k T={w['T']} H={w['H']} d={w['d']} block={w['block']} plan="
        f"{la.la_prefill_plan(w['T'], 1, w['H'], w['d'], w['block'], la.LA_BF16)}")
    o, kv = run_gpu(w["q"], w["k"], w["v"], w["cu"], w["block"])
    check_against_oracle(w["q"], w["k"], w["v"], w["cu"], o, kv, False, "prefill_8k")
    # the last output equals q_last . final state (links the two outputs)
    q_last = as_f64(w["q"][-1])
    o_last = np.einsum("hi,hij->hj", q_last, kv[0].astype(np.float64))
    ErrAcc().add(o[-1], o_last).check(False, "last-token identity")


SUPPORTED = [(d, b, dt) for d in (16, 32, 64, 128) for b in (32, 64, 128) for dt in ("bf16", "fp32")
             if not (dt == "fp32" and d >= 64 and b == 128)]


@pytest.mark.parametrize("d,block,dtype", SUPPORTED, ids=[f"d{d}-b{b}-{t}" for d, b, t in SUPPORTED])
def test_shapes_ragged(d, block, dtype):
    T, H = 1000, 3
    q, k, v = rand_inputs(7 + d + block, T, H, d, dtype)
    cu = np.array([0, 1, 1, 200, 611, 1000], dtype=np.int32)
    log(f"  d={d} block={block} {dtype} T={T} cu={cu.tolist()}")
    o, kv = run_gpu(q, k, v, cu, block)
    check_against_oracle(q, k, v, cu, o, kv, dtype == "fp32", f"d{d} b{block} {dtype}")


SPLITS = [dict(seg_len=64, value_slices=1), dict(seg_len=64, value_slices=4, force_scan=True),
          dict(seg_len=192, value_slices=2), dict(seg_len=128, value_slices=4), dict(seg_len=640, value_slices=1),
          dict(seg_len=64, value_slices=2, force_scan=False)]


@pytest.mark.parametrize("opts", SPLITS, ids=[str(s) for s in SPLITS])
def test_segment_splitting(opts):
    T, H, d, block = 2000, 2, 128, 64
    q, k, v = rand_inputs(31, T, H, d, "bf16")
    cu = np.array([0, 700, 700, 701, 1500, 1563, 2000], dtype=np.int32)
    plan = la.la_prefill_plan(T, len(cu) - 1, H, d, block, la.LA_BF16, la.make_opts(**opts))
    log(f"  split {opts} plan={plan}")
    o, kv = run_gpu(q, k, v, cu, block, **opts)
    check_against_oracle(q, k, v, cu, o, kv, False, f"split {opts}")


PIECE_CASES = [(d, block, dtype, opts)
               for d, block, dtype in ((128, 64, "bf16"), (64, 64, "bf16"), (32, 64, "bf16"), (128, 128, "bf16"),
                                       (128, 32, "fp32"), (16, 32, "fp32"))
               for opts in (dict(seg_len=128), dict(seg_len=256, value_slices=2), dict(seg_len=640))]


@pytest.mark.parametrize("d,block,dtype,opts", PIECE_CASES,
                         ids=[f"d{c[0]}-b{c[1]}-{c[2]}-{c[3]}" for c in PIECE_CASES])
def test_document_pieces(d, block, dtype, opts):
    """The document-piece work list: documents longer than the piece length
    are cut into several pieces (their earlier pieces' states summed in the
    prologue), empty documents get units of their own, the planning kernel
    orders the pieces longest first.  Against the oracle, with incoming states."""
    import torch

    if opts["seg_len"] % block:
        pytest.skip("piece length not a multiple of the block")
    lens = [0, 1500, 3, 0, 0, 200, 1, 777, 129, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H = int(cu[-1]), 3
    dt = la.LA_BF16 if dtype == "bf16" else la.LA_FP32
    S = opts.get("value_slices", 0)
    try:
        plan = la.la_prefill_plan(T, len(lens), H, d, block, dt, la.make_opts(work_list=2, **opts))
    except la.LAError:
        pytest.skip("this slicing does not fit LDS for this shape")
    assert plan["packed"] == 1
    log(f"  pieces d={d} b={block} {dtype} {opts} plan={plan}")
    q, k, v = rand_inputs(171 + d + block, T, H, d, dtype)
    kv_in = np.ascontiguousarray(la_inputs.normal(172, 7, (len(lens), H, d, d), "fp32", float(np.sqrt(2000)) / d),
                                 dtype=np.float32)
    o, kv = la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(cu), block=block, work_list=2,
                       kv_state_in=to_dev(kv_in), **opts)
    torch.cuda.synchronize()
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu, kv_in=kv_in)
    ErrAcc().add(to_host(o), o_ref).check(dtype == "fp32", f"pieces {opts} o")
    ErrAcc().add(to_host(kv), kv_ref).check(dtype == "fp32", f"pieces {opts} kv_state")
    # the empty documents' final states are their incoming states, exactly
    kvh = to_host(kv)
    for i, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(kvh[i], kv_in[i])


SLOT_CASES = [(S, opts) for S in (1, 2)
              for opts in (dict(), dict(seg_len=64), dict(seg_len=192, force_scan=True), dict(seg_len=1024))]


@pytest.mark.parametrize("S,opts", SLOT_CASES, ids=[f"S{S}-{o}" for S, o in SLOT_CASES])
def test_three_tile_slots(S, opts):
    """The transpose-read loop loading two blocks ahead (three tile slots)
    on ragged packed documents, with incoming states: against the oracle,
    and bit for bit against two slots (the per-block arithmetic is the same)."""
    import torch

    lens = [5, 0, 295, 1, 699, 64, 0, 1436, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 3, 128
    q, k, v = rand_inputs(141, T, H, d, "bf16")
    kv_in = np.ascontiguousarray(la_inputs.normal(142, 7, (len(lens), H, d, d), "fp32", float(np.sqrt(2000)) / d),
                                 dtype=np.float32)
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu, kv_in=kv_in)
    outs = []
    for slots in (3, 2):
        plan = la.la_prefill_plan(T, len(lens), H, d, 64, la.LA_BF16, la.make_opts(value_slices=S, slots=slots, **opts))
        assert plan["slots"] == slots and plan["variant"] == 2
        log(f"  slots={slots} S={S} {opts} plan={plan}")
        o, kv = la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(cu), block=64, value_slices=S, slots=slots,
                           kv_state_in=to_dev(kv_in), **opts)
        torch.cuda.synchronize()
        o, kv = to_host(o), to_host(kv)
        ErrAcc().add(o, o_ref).check(False, f"slots {slots} o")
        ErrAcc().add(kv, kv_ref).check(False, f"slots {slots} kv_state")
        outs.append((o, kv))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


VARIANT_CASES = [(d, S, opts) for d, slices in ((128, (1, 2)), (64, (1,))) for S in slices
                 for opts in (dict(), dict(seg_len=64, force_scan=True), dict(seg_len=192), dict(seg_len=64))]


@pytest.mark.parametrize("d,S,opts", VARIANT_CASES, ids=[f"d{d}-S{S}-{o}" for d, S, o in VARIANT_CASES])
def test_block_loop_variants(d, S, opts):
    """The transpose-read loop (variant 2) and the generic loop (variant 1)
    on ragged packed documents, with and without segment splitting."""
    T, H, block = 1500, 3, 64
    q, k, v = rand_inputs(61 + d, T, H, d, "bf16")
    cu = np.array([0, 5, 5, 300, 301, 1000, 1064, 1500], dtype=np.int32)
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu)
    outs = []
    for variant in (1, 2):
        log(f"  variant {variant} d={d} S={S} {opts}")
        o, kv = run_gpu(q, k, v, cu, block, value_slices=S, variant=variant, **opts)
        ErrAcc().add(o, o_ref).check(False, f"variant {variant} o")
        ErrAcc().add(kv, kv_ref).check(False, f"variant {variant} kv_state")
        outs.append((o, kv))
    # the two loops round the same products the same way: outputs agree closely
    ErrAcc().add(outs[1][0], as_f64(outs[0][0])).check(False, "variant 2 vs 1")


B128_CASES = [(d, opts) for d in (128, 64)
              for opts in (dict(), dict(seg_len=128, force_scan=True), dict(seg_len=256), dict(seg_len=384),
                           dict(seg_len=640, work_list=2))]
B128_CASES += [(128, dict(value_slices=2, **o)) for o in (dict(), dict(seg_len=128, force_scan=True),
                                                         dict(seg_len=384), dict(seg_len=640, work_list=2))]


@pytest.mark.parametrize("d,opts", B128_CASES, ids=[f"d{d}-{o}" for d, o in B128_CASES])
def test_block128_loop(d, opts):
    """128-token blocks on the transpose-read loop (two 64-row halves per
    block, the second with its cross term against the first's keys, one state
    update per block), with 64-column slices and at full width, on documents
    whose lengths leave every kind of last block: one half, one and a bit, two
    full halves, with and without segment splitting, the scan and document
    pieces; against the oracle and against the generic loop at block 128."""
    lens = [1, 63, 64, 65, 0, 127, 128, 129, 191, 192, 193, 0, 700, 257, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H = int(cu[-1]), 3
    q, k, v = rand_inputs(71 + d, T, H, d, "bf16")
    kv_in = np.ascontiguousarray(la_inputs.normal(72, 7, (len(lens), H, d, d), "fp32", float(np.sqrt(300)) / d),
                                 dtype=np.float32)
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu, kv_in=kv_in)
    plan = la.la_prefill_plan(T, len(lens), H, d, 128, la.LA_BF16, la.make_opts(**opts))
    log(f"  block 128 d={d} {opts} plan={plan}")
    assert plan["variant"] == 2 and plan["slots"] == 3
    outs = []
    for variant in (2, 1):
        # (the generic loop takes its own slicing: full width does not fit its tiles at 128 tokens)
        vo = opts if variant == 2 else {k2: x for k2, x in opts.items() if k2 != "value_slices"}
        o, kv = run_gpu(q, k, v, cu, 128, kv_state_in=to_dev(kv_in), variant=variant, **vo)
        ErrAcc().add(o, o_ref).check(False, f"b128 variant {variant} o")
        ErrAcc().add(kv, kv_ref).check(False, f"b128 variant {variant} kv_state")
        outs.append(o)
    ErrAcc().add(outs[0], as_f64(outs[1])).check(False, "b128 transpose-read vs generic")
    # run to run: the same bits
    o2, _ = run_gpu(q, k, v, cu, 128, kv_state_in=to_dev(kv_in), **opts)
    assert np.array_equal(o2, outs[0])


def test_varlen_tails_and_empty_docs():
    lens = [1, 63, 64, 65, 0, 127, 128, 129, 0, 300, 1, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 4, 64
    q, k, v = rand_inputs(41, T, H, d, "bf16")
    for block in (32, 64, 128):
        for opts in (dict(), dict(seg_len=block, value_slices=2), dict(seg_len=max(64, block), work_list=2)):
            log(f"  tails block={block} {opts}")
            o, kv = run_gpu(q, k, v, cu, block, **opts)
            o_ref, kv_ref = check_against_oracle(q, k, v, cu, o, kv, False, f"tails b{block} {opts}")
            for i, n in enumerate(lens):
                if n == 0:
                    assert np.all(kv[i] == 0.0)
    # packed == separate runs, bit for bit, when neither is cut into segments
    # (segment cuts sit at packed-token offsets, so they would fall at
    # different document offsets in the two runs and change summation order)
    one = dict(seg_len=1024)
    assert T <= one["seg_len"]
    o_all, kv_all = run_gpu(q, k, v, cu, 64, **one)
    for i, n in enumerate(lens):
        if n == 0:
            continue
        a, b = cu[i], cu[i + 1]
        oi, kvi = run_gpu(q[a:b], k[a:b], v[a:b], np.array([0, n], np.int32), 64, **one)
        assert np.array_equal(oi, o_all[a:b]) and np.array_equal(kvi[0], kv_all[i])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [16, 128])
def test_exact_integer_inputs_bitexact(dtype, d):
    """Entries in {-1, 0, 1} and at most 256 tokens per document: every partial
    sum is an integer below 2^24 and every bf16 operand (scores <= d, states <=
    256) is exact, so any blocking gives the exact result."""
    T, H = 256, 2
    q, k, v = (la_inputs.ternary(77, i, (T, H, d), dtype) for i in range(3))
    cu = np.array([0, 100, 256], dtype=np.int32)
    o_ref, kv_ref = oracle.recurrent(q, k, v, cu)
    assert np.all(o_ref == np.round(o_ref)) and np.max(np.abs(o_ref)) < 2 ** 24
    blocks = (32, 64, 128) if not (dtype == "fp32" and d >= 64) else (32, 64)
    for block in blocks:
        for opts in (dict(), dict(seg_len=block, value_slices=1), dict(seg_len=block, value_slices=d // 32 or 1),
                     dict(seg_len=block, work_list=2)):
            try:
                la.la_prefill_plan(T, 2, H, d, block, la.LA_BF16 if dtype == "bf16" else la.LA_FP32,
                                   la.make_opts(**opts))
            except la.LAError:
                continue  # this slicing does not fit LDS for this shape
            log(f"  exact {dtype} d={d} block={block} {opts}")
            o, kv = run_gpu(q, k, v, cu, block, **opts)
            if dtype == "bf16":
                assert np.array_equal(o, bf16_rne_from_f64(o_ref))
            else:
                assert np.array_equal(o.astype(np.float64), o_ref)
            assert np.array_equal(kv.astype(np.float64), kv_ref)


def test_run_to_run_bitwise_determinism():
    w = la_inputs.prefill_inputs("prefill_8k")
    first = run_gpu(w["q"], w["k"], w["v"], w["cu"], 64)
    for _ in range(4):
        again = run_gpu(w["q"], w["k"], w["v"], w["cu"], 64)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


def test_stale_hip_error_not_reported():
    """An error an earlier HIP call left in the thread's last-error slot (here
    a host-side query of a device index that does not exist) is neither
    reported by the library's calls nor cleared by them.  Every buffer is
    allocated before the error is planted (torch's allocator would report it)."""
    import torch

    hip = ctypes.CDLL("libamdhip64.so")
    for f in ("hipGetLastError", "hipPeekAtLastError", "hipDeviceGetAttribute", "hipDeviceSynchronize"):
        getattr(hip, f).restype = ctypes.c_int
    T, H, d = 1000, 2, 128
    q, k, v = rand_inputs(56, T, H, d, "bf16")
    cu = np.array([0, 400, 1000], dtype=np.int32)
    qd, kd, vd, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(cu)
    o = torch.empty_like(qd)
    kv = torch.empty((2, H, d, d), dtype=torch.float32, device="cuda")
    plan = la.la_prefill_plan(T, 2, H, d, 64, la.LA_BF16, la.make_opts(seg_len=256))
    assert plan["num_segments"] > 1  # segment states, look-back and block loop all launch
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
    s0 = la_inputs.normal(56, 9, (2, H, d, d), "fp32", 0.01)
    sd = to_dev(s0)
    q2, k2, v2 = to_dev(q[:2]), to_dev(k[:2]), to_dev(v[:2])
    o2 = torch.empty_like(q2)
    torch.cuda.synchronize()
    hip.hipGetLastError()  # start from a clean slot
    value = ctypes.c_int(0)
    assert hip.hipDeviceGetAttribute(ctypes.byref(value), 0, 1 << 20) != 0  # no such device
    stale = hip.hipPeekAtLastError()
    assert stale != 0
    try:
        la.prefill(qd, kd, vd, cud, block=64, out=o, kv_state_out=kv, workspace=ws, seg_len=256)
        la.decode(q2, k2, v2, sd, out=o2)
        assert hip.hipDeviceSynchronize() == 0
        assert hip.hipPeekAtLastError() == stale
    finally:
        hip.hipGetLastError()
    check_against_oracle(q, k, v, cu, to_host(o), to_host(kv), False, "after a stale HIP error")
    s_ref = s0.astype(np.float64).reshape(-1, d, d)
    o_ref = oracle.decode_step(q[:2].reshape(-1, d), k[:2].reshape(-1, d), v[:2].reshape(-1, d), s_ref)
    ErrAcc().add(to_host(o2).reshape(-1, d), o_ref).check(False, "decode o after a stale HIP error")
    ErrAcc().add(to_host(sd).reshape(-1, d, d), s_ref).check(True, "decode state after a stale HIP error")


def test_guard_bands():
    """Outputs are written exactly inside their bounds."""
    import torch

    T, H, d, block = 777, 3, 128, 64
    q, k, v = rand_inputs(55, T, H, d, "bf16")
    cu = np.array([0, 300, 777], dtype=np.int32)
    guard = 4096
    n_o = T * H * d
    n_kv = 2 * H * d * d
    o_buf = torch.full((n_o + 2 * guard,), 1.5, dtype=torch.bfloat16, device="cuda")
    kv_buf = torch.full((n_kv + 2 * guard,), -7.25, dtype=torch.float32, device="cuda")
    o_view = o_buf[guard:guard + n_o].view(T, H, d)
    kv_view = kv_buf[guard:guard + n_kv].view(2, H, d, d)
    for opts in (dict(), dict(seg_len=64, value_slices=4), dict(seg_len=64, work_list=2)):
        la.prefill(to_dev(q), to_dev(k), to_dev(v), to_dev(cu), block=block, out=o_view, kv_state_out=kv_view,
                   **opts)
        torch.cuda.synchronize()
        ob = o_buf.float().cpu().numpy()
        kb = kv_buf.cpu().numpy()
        assert np.all(ob[:guard] == 1.5) and np.all(ob[guard + n_o:] == 1.5)
        assert np.all(kb[:guard] == -7.25) and np.all(kb[guard + n_kv:] == -7.25)
        ErrAcc().add(to_host(o_view), oracle.recurrent(q, k, v, cu)[0]).check(False, f"guarded o {opts}")


def test_zero_tokens():
    import torch

    H, d = 2, 64
    buf = torch.zeros((1, H, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full((1, H, d), 3.0, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    kv = torch.full((3, H, d, d), 9.0, dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = la.la_prefill(p(buf), p(buf), p(buf), p(o), p(cu), H, d, 64, p(kv), 3, 0, la.LA_BF16, None, 0,
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == la.LA_OK
    torch.cuda.synchronize()
    assert torch.all(kv == 0).item()
    assert torch.all(o == 3.0).item()  # nothing written


def _full_compare(w, block, head_group, **opts):
    import torch

    T, H, d = w["T"], w["H"], w["d"]
    plan = la.la_prefill_plan(T, len(w["cu"]) - 1, H, d, block, la.LA_BF16, la.make_opts(**opts))
    log(f"  full T={T} H={H} block={block} docs={len(w['cu']) - 1} plan={plan}")
    o, kv = run_gpu(w["q"], w["k"], w["v"], w["cu"], block, **opts)
    torch.cuda.empty_cache()
    acc_o, acc_kv = ErrAcc(), ErrAcc()
    for h0 in range(0, H, head_group):
        h1 = min(H, h0 + head_group)
        o_ref, kv_ref = oracle.recurrent(w["q"], w["k"], w["v"], w["cu"], heads=(h0, h1))
        acc_o.add(o[:, h0:h1], o_ref)
        acc_kv.add(kv[:, h0:h1], kv_ref[:, h0:h1])
        log(f"    heads {h0}..{h1 - 1} compared")
        del o_ref
    acc_o.check(False, "o")
    acc_kv.check(False, "kv_state")


def test_full_varlen_128k():
    w = la_inputs.prefill_inputs("varlen_128k")
    _full_compare(w, 64, 8)


@pytest.mark.parametrize("block", [64, 128])
def test_full_long_1m(block):
    w = la_inputs.prefill_inputs("long_1m")
    _full_compare(w, block, 4)
