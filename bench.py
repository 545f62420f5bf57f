#!/usr/bin/env python3
"""Benchmark: causal linear attention (Lightning-style) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_1m]

A step is one pass of the hot path over one batch of synthetic input: one
la_prefill call over the whole workload (segment states, prefix scan when the
plan needs one, block loop).  The headline workload is the 8-head x
1,048,576-token bf16 prefill (d = 128, block 64), the largest of the
single-GPU prefill workloads.  Inputs are generated on the host from fixed
seeds and copied to HBM before timing; small workloads rotate over several
input sets so that the timed steps read HBM rather than the 256 MB last-level
cache.

`value` comes from a timed loop of K steps with nothing but the calls in it
(synchronised before and after).  A second loop over the same steps launches
the block-loop kernel through hipExtLaunchKernel with start/end events on the
launch stream: `roofline` is that kernel's algorithmic bytes (q, k, v read + o
written, 8 d bytes per token-head) over its average duration.  `whole_call`
is the same bytes over the whole step (every kernel of the call), the figure
the 60 % target is stated for.  Both are also given against `ceilings`:
contiguous HBM streams written here (include/la_bench.h) timed in the same
run, 3 reads + 1 write for prefill and 1 read + 1 write for decode.

Reported beside the headline, in the same line: the packed-document and 8k
prefill workloads (`workloads`, the packed one also at block 128), the
headline workload at block 128 and with
the decayed variant (`long_1m_block128`, `decay`), the prefill's backward and a
forward + backward training step on the headline workload (`backward`), the
decode workload (256 sequences x 64 heads, fp32 state, 1000 steps, `decode`,
with its decayed step), and `cpu_baseline`: the fp64 oracle (recurrent form)
on the host cores over a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
DECODE_SAMPLE = {}  # host copy of a few decode states for the oracle's timing

KERNEL_SOURCES = ["la_prefill_kernels.h", "la_prefill_v2.h", "la_device.h", "la_tiles.h", "la_prefill_launch.inl",
                  "la_prefill_bf16.hip", "la_host.cpp"]
MAIN_KERNEL = {1: "la_prefill_main_kernel", 2: "la_prefill_main_v2"}  # by the plan's block-loop variant


def main_kernel(plan: dict, block: int) -> str:
    """The block-loop kernel a plan runs (128-token blocks have a transpose-read loop of their own)."""
    return "la_prefill_main_v2_b128" if plan["variant"] == 2 and block == 128 else MAIN_KERNEL[plan["variant"]]
DECODE_SOURCES = ["la_decode_kernels.h", "la_device.h", "la_decode.hip"]
METRIC = "prefill tokens·heads/s (bf16, d=128) + % roofline; decode steps/s"
GIB = 1 << 30


def sources_sha(names) -> str:
    """Hash of the kernel sources' code (// comments and blank lines left
    out, so that a comment edit does not orphan the counter summaries)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "causal_linear_attention_la_amd", "csrc", n), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


class Hip:
    """hipEvent helpers through the HIP runtime (events on the launch stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e

    def record(self, e, stream_ptr):
        rc = self.lib.hipEventRecord(e, ctypes.c_void_p(stream_ptr))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def gpu_time(torch, hip, fn, reps: int) -> float:
    """Seconds per call of fn() over reps calls, by one event pair on the
    current stream around all of them (after one untimed call)."""
    stream = torch.cuda.current_stream().cuda_stream
    fn()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(reps):
        fn()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    s = hip.elapsed_ms(e0, e1) / 1e3 / reps
    hip.destroy(e0)
    hip.destroy(e1)
    return s


def load_traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ ceilings

def stream_ceilings(la, torch, hip) -> dict:
    """Bandwidth (GB/s of bytes read + written) of the contiguous streams in
    la_bench_stream over 1 GiB per source: the best of 128 to 65536
    workgroups (up to a few resident per CU, as the decode step runs, and
    beyond), plain and non-temporal accesses, two rounds of 20 passes."""
    lib = la.load()
    bufs = [torch.empty(GIB, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(4)]
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    for mode, name, nbytes in ((0, "copy_1r1w", 2 * GIB), (1, "stream_3r1w", 4 * GIB)):
        best, how = 0.0, None
        for _ in range(2):
            for wgs in (128, 256, 512, 1024, 2048, 4096, 16384, 65536):
                for nt in (0, 1):
                    def fn():
                        st = lib.la_bench_stream(mode, P(bufs[0]), P(bufs[1]), P(bufs[2]), P(bufs[3]), GIB, wgs, nt,
                                                 sp)
                        if st != 0:
                            raise RuntimeError(f"la_bench_stream: {st}")
                    gbs = nbytes / gpu_time(torch, hip, fn, 20) / 1e9
                    if gbs > best:
                        best, how = gbs, f"{wgs} workgroups, {'non-temporal' if nt else 'plain'} accesses"
        out[name] = {"GBs": best, "config": how}
    del bufs
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------- prefill

def device_sets(torch, w, rotate: int):
    """Input set 0 is the seeded workload; the others are copies shifted by
    one token per set (same statistics, different bytes in HBM)."""
    T, H, d = w["T"], w["H"], w["d"]

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    per_set = 4 * T * H * d * (2 if w["dtype"] == "bf16" else 4)
    nsets = max(1, min(rotate, int((8 * GIB) // max(per_set, 1))))
    q0, k0, v0 = dev(w["q"]), dev(w["k"]), dev(w["v"])
    sets = []
    for i in range(nsets):
        sh = i % max(T, 1)
        q, k, v = (torch.roll(x, sh, 0).contiguous() if sh else x for x in (q0, k0, v0))
        sets.append((q, k, v, torch.empty_like(q)))
    return sets


def bench_prefill(name, args, la, torch, hip, steps: int, warmup: int, graph: bool, keep_sets: bool = False):
    """One prefill workload: clean timed loop (value), event-stamped loop
    (block-loop kernel duration), optionally HIP-graph replay."""
    import la_inputs

    w = la_inputs.prefill_inputs(name)
    w["name"] = name
    T, H, d, block = w["T"], w["H"], w["d"], args.block or w["block"]
    dt = la.LA_BF16 if w["dtype"] == "bf16" else la.LA_FP32
    num_seqs = len(w["cu"]) - 1
    opts = dict(seg_len=args.seg_len, value_slices=args.slices, force_scan=args.force_scan, slots=args.slots)
    plan = la.la_prefill_plan(T, num_seqs, H, d, block, dt, la.make_opts(**opts))
    sets = device_sets(torch, w, args.rotate)
    nsets = len(sets)
    cu = torch.from_numpy(w["cu"]).cuda()
    kv = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i, ev0=None, ev1=None):
        q, k, v, o = sets[i % nsets]
        la.prefill(q, k, v, cu, block=block, out=o, kv_state_out=kv, workspace=ws, begin_event=ev0, end_event=ev1,
                   **opts)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed loop: the calls and nothing else
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(e0, sp)
    for i in range(steps):
        step(i)
    hip.record(e1, sp)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_s = hip.elapsed_ms(e0, e1) / 1e3
    hip.destroy(e0)
    hip.destroy(e1)

    # the same steps again, the block-loop kernel of each launched with events
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, evs[i][0], evs[i][1])
    torch.cuda.synchronize()
    kernel_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)

    graph_value = None
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            step(0)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for i in range(nsets):
                    step(i)
        torch.cuda.synchronize()
        reps = max(1, steps // nsets)
        g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        graph_value = T * H * nsets * reps / (time.perf_counter() - t1)
        del g

    esz = 2 if w["dtype"] == "bf16" else 4
    algo_bytes = T * H * 4 * d * esz  # q, k, v read + o written
    avg_kernel_s = float(np.mean(kernel_ms)) / 1e3
    achieved = algo_bytes / avg_kernel_s / 1e9
    sha = sources_sha(KERNEL_SOURCES)
    kname = main_kernel(plan, block)
    roof_th = HBM_PEAK_GBS * 1e9 / (algo_bytes / (T * H))  # token-heads/s with every byte at HBM peak
    value = T * H * steps / elapsed
    rec = {
        "workload": name, "value": value, "unit": "token·heads/s", "steps": steps, "warmup": warmup,
        "ms_per_step": elapsed / steps * 1e3, "gpu_ms_per_step": gpu_s / steps * 1e3,
        "config": {"workload": name, "documents": num_seqs, "heads": H, "tokens": T, "head_dim": d, "block": block,
                   "dtype": w["dtype"], "seg_len": plan["seg_len"], "value_slices": plan["value_slices"],
                   "segments": plan["num_segments"], "scan": plan["scan"], "slots": plan["slots"],
                   "workgroups": plan["units"], "input_sets": nsets},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(kname, name, sha),
                     "kernel_ms": avg_kernel_s * 1e3, "kernel_launches_timed": steps,
                     "algorithmic_bytes": algo_bytes, "kernel_sources_sha": sha},
        "whole_call": {"achieved": algo_bytes * steps / elapsed / 1e9, "unit": "GB/s",
                       "roofline_token_heads_per_s": roof_th, "frac": value / roof_th},
        "graph_replay_value": graph_value,
    }
    rec["roofline"]["whole_call_frac"] = rec["whole_call"]["frac"]
    # outputs of the seeded input set, for the error against the oracle (copies:
    # later measurements reuse these buffers)
    step(0)
    torch.cuda.synchronize()
    w["gpu_o"] = sets[0][3].clone()
    w["gpu_kv"] = kv.clone()
    if keep_sets:
        w["dev_sets"] = sets
    return rec, w


def bench_block(la, torch, hip, w, block: int, steps: int) -> dict:
    """The same workload and device inputs with another block size: whole-call
    time and the block-loop kernel's duration (events), plan included."""
    T, H, d = w["T"], w["H"], w["d"]
    num_seqs = len(w["cu"]) - 1
    dt = la.LA_BF16 if w["dtype"] == "bf16" else la.LA_FP32
    plan = la.la_prefill_plan(T, num_seqs, H, d, block, dt)
    q, k, v, o = w["dev_sets"][0]
    cu = torch.from_numpy(w["cu"]).cuda()
    kv = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
    call = lambda: la.prefill(q, k, v, cu, block=block, out=o, kv_state_out=kv, workspace=ws)
    s = gpu_time(torch, hip, call, steps)
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    for a, b in evs:
        la.prefill(q, k, v, cu, block=block, out=o, kv_state_out=kv, workspace=ws, begin_event=a, end_event=b)
    torch.cuda.synchronize()
    kms = float(np.mean([hip.elapsed_ms(a, b) for a, b in evs]))
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    algo = T * H * 8 * d
    roof_th = HBM_PEAK_GBS * 1e9 / (8 * d)
    return {"workload": w["name"], "block": block, "value": T * H / s, "unit": "token·heads/s",
            "gpu_ms_per_step": s * 1e3, "steps": steps,
            "plan": {k2: plan[k2] for k2 in ("seg_len", "value_slices", "num_segments", "scan", "variant", "units")},
            "block_loop": {"kernel": main_kernel(plan, block), "kernel_ms": kms,
                           "frac": algo / (kms / 1e3) / 1e9 / HBM_PEAK_GBS},
            "whole_call_frac": T * H / s / roof_th}


def bench_decay(la, torch, hip, w, steps: int) -> dict:
    """The decayed variant (la_prefill_decay) on the same workload and device
    inputs, per-head factors lambda_h = 1 - 2^-(5 + h): whole call and the
    block-loop kernel (events)."""
    T, H, d = w["T"], w["H"], w["d"]
    num_seqs = len(w["cu"]) - 1
    dt = la.LA_BF16 if w["dtype"] == "bf16" else la.LA_FP32
    plan = la.la_prefill_plan(T, num_seqs, H, d, 64, dt)
    q, k, v, o = w["dev_sets"][0]
    cu = torch.from_numpy(w["cu"]).cuda()
    kv = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
    lam = torch.tensor([1.0 - 2.0 ** -(5 + h) for h in range(H)], dtype=torch.float32, device="cuda")
    call = lambda a=None, b=None: la.prefill(q, k, v, cu, block=64, out=o, kv_state_out=kv, workspace=ws, decay=lam,
                                             begin_event=a, end_event=b)
    s = gpu_time(torch, hip, call, steps)
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    for a, b in evs:
        call(a, b)
    torch.cuda.synchronize()
    kms = float(np.mean([hip.elapsed_ms(a, b) for a, b in evs]))
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    algo = T * H * 8 * d
    roof_th = HBM_PEAK_GBS * 1e9 / (8 * d)
    return {"workload": w["name"], "lambda": "1 - 2^-(5 + h)", "value": T * H / s, "unit": "token·heads/s",
            "gpu_ms_per_step": s * 1e3, "steps": steps,
            "block_loop": {"kernel": main_kernel(plan, 64), "kernel_ms": kms,
                           "frac": algo / (kms / 1e3) / 1e9 / HBM_PEAK_GBS},
            "whole_call_frac": T * H / s / roof_th}


def with_ceiling(roof: dict, ceiling_gbs: float):
    roof["measured_ceiling_GBs"] = ceiling_gbs
    roof["frac_of_measured_ceiling"] = roof["achieved"] / ceiling_gbs


# ------------------------------------------------------------------ backward

def bench_backward(args, la, torch, hip, w, dev_sets, steps: int):
    """la_prefill_backward over the same workload: dq, dk, dv from dO with no
    incoming state and no final-state gradient.  Algorithmic bytes per call:
    q, k, v, dO read and dq, dk, dv written once, 14 d bytes per token-head
    in bf16.  Timed with one event pair on the launch stream around all calls.
    Then a training step's attention work: the forward, and the backward handed
    the forward's workspace (of the backward's size, la_prefill_backward_workspace_size,
    so that the backward's dv and dk passes share a launch)."""
    import la_inputs

    T, H, d = w["T"], w["H"], w["d"]
    esz = 2 if w["dtype"] == "bf16" else 4
    block = args.block or w["block"]
    opts = dict(seg_len=args.seg_len, value_slices=args.slices, force_scan=args.force_scan, slots=args.slots)
    cu = torch.from_numpy(w["cu"]).cuda()
    d0 = la_inputs.normal(la_inputs.WORKLOADS[w["name"]]["seed"], 8, (T, H, d), w["dtype"], 1.0)
    dout0 = torch.from_numpy(d0.view(np.int16)).view(torch.bfloat16).cuda() if d0.dtype == np.uint16 \
        else torch.from_numpy(d0).cuda()
    del d0
    sets = []
    for i, (q, k, v, _) in enumerate(dev_sets):
        dout = torch.roll(dout0, i, 0).contiguous() if i else dout0
        sets.append((q, k, v, dout))
    outs = (torch.empty_like(dout0), torch.empty_like(dout0), torch.empty_like(dout0), None)
    num_seqs = len(w["cu"]) - 1
    dt = la.LA_BF16 if w["dtype"] == "bf16" else la.LA_FP32
    # the backward's workspace size: room for the transposed segment states, so
    # the dv and dk passes share a launch (the forward uses a prefix of it)
    need = la.la_prefill_backward_workspace_size(T, num_seqs, H, d, block, dt, la.make_opts(**opts))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    it = [0]

    def call():
        q, k, v, dout = sets[it[0] % len(sets)]
        it[0] += 1
        la.backward(q, k, v, dout, cu, block=block, want_dkv_in=False, workspace=ws, out=outs, **opts)

    s = gpu_time(torch, hip, call, steps)
    algo = T * H * 7 * d * esz
    achieved = algo / s / 1e9
    rec = {"workload": w["name"], "value": T * H / s, "unit": "token·heads/s", "steps": steps,
           "gpu_ms_per_step": s * 1e3,
           "roofline": {"bound": "hbm", "kernel": "la_prefill_backward (whole call)", "achieved": achieved,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                        "algorithmic_bytes": algo}}
    fo = torch.empty_like(dout0)
    fkv = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device="cuda")

    def train():
        q, k, v, dout = sets[it[0] % len(sets)]
        it[0] += 1
        la.prefill(q, k, v, cu, block=block, out=fo, kv_state_out=fkv, workspace=ws, **opts)
        la.backward(q, k, v, dout, cu, block=block, want_dkv_in=False, out=outs, forward_workspace=ws, **opts)

    s = gpu_time(torch, hip, train, steps)
    talgo = T * H * 11 * d * esz  # forward 8d + backward 14d bytes per token-head (bf16)
    tach = talgo / s / 1e9
    rec["train_step"] = {"value": T * H / s, "unit": "token·heads/s", "gpu_ms_per_step": s * 1e3,
                         "roofline": {"bound": "hbm", "achieved": tach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": tach / HBM_PEAK_GBS, "algorithmic_bytes": talgo}}
    del sets, outs, ws, fo, dout0
    torch.cuda.empty_cache()
    return rec


# -------------------------------------------------------------------- decode

def bench_decode(args, la, torch, hip):
    import la_inputs

    cfg = la_inputs.WORKLOADS["decode_256x64"]
    ns, H, d, seed, pool = cfg["num_seqs"], cfg["H"], cfg["d"], cfg["seed"], cfg["pool"]
    lo, hi = cfg["prefix"]
    steps = args.decode_steps
    S0 = la_inputs.decode_states(seed, ns, H, d, lo, hi)
    S = torch.from_numpy(S0.reshape(ns, H, d, d)).cuda()
    DECODE_SAMPLE["S"] = S0[: 8 * H].copy()  # the first 8 sequences, for the oracle's timing
    del S0
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    sets = [tuple(dev(x) for x in la_inputs.decode_step_inputs(seed, s, ns, H, d, "bf16")) for s in range(pool)]
    o = torch.empty((ns, H, d), dtype=torch.bfloat16, device="cuda")
    for i in range(10):
        la.decode(*sets[i % pool], S, out=o)
    torch.cuda.synchronize()
    sp = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(e0, sp)
    for i in range(steps):
        la.decode(*sets[i % pool], S, out=o)
    hip.record(e1, sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = hip.elapsed_ms(e0, e1) / 1e3
    hip.destroy(e0)
    hip.destroy(e1)
    bytes_step = ns * H * (2 * d * d * 4 + 4 * d * 2)
    achieved = bytes_step * steps / gpu_s / 1e9
    # the decayed step (la_decode_decay), per-head factors 1 - 2^-(5 + h mod 8)
    lam = torch.tensor([1.0 - 2.0 ** -(5 + h % 8) for h in range(H)], dtype=torch.float32, device="cuda")
    it = [0]

    def dstep():
        la.decode(*sets[it[0] % pool], S, out=o, decay=lam)
        it[0] += 1

    dec_s = gpu_time(torch, hip, dstep, 200)
    del S, sets, o
    torch.cuda.empty_cache()
    return {"workload": "decode_256x64", "value": steps / wall, "unit": "steps/s", "steps": steps,
            "ms_per_step": wall / steps * 1e3, "gpu_ms_per_step": gpu_s / steps * 1e3,
            "roofline": {"bound": "hbm", "kernel": "la_decode_kernel", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "bytes_per_step": bytes_step,
                         "kernel_sources_sha": sources_sha(DECODE_SOURCES)},
            "decay": {"gpu_ms_per_step": dec_s * 1e3, "value": 1.0 / dec_s, "unit": "steps/s", "steps": 200,
                      "frac": bytes_step / dec_s / 1e9 / HBM_PEAK_GBS}}


# -------------------------------------------------------------- CPU baseline

def error_vs_oracle(gpu, ref) -> tuple:
    g = np.asarray(gpu, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    den = max(float(np.linalg.norm(r)), 1e-300)
    return float(np.linalg.norm(g - r) / den), float(np.max(np.abs(g - r)) / max(float(np.max(np.abs(r))), 1e-300))


def cpu_baseline(w, target_cpu_s: float = 12.0) -> dict:
    """The fp64 oracle as it stands (recurrent form, all host threads) on a
    bounded sample of the workload: its first Ts tokens of every head (for a
    one-document workload, exactly the first Ts outputs of the full call),
    repeated until about target_cpu_s seconds of CPU time are spent.  The GPU
    outputs of those tokens are compared with the oracle's."""
    import oracle

    oracle.build()
    T, H = w["T"], w["H"]
    one_doc = len(w["cu"]) == 2
    Ts = min(T, 131072) if one_doc else T
    cu = np.array([0, Ts], dtype=np.int32) if one_doc else w["cu"]
    q, k, v = (np.ascontiguousarray(w[x][:Ts]) for x in ("q", "k", "v"))
    reps, wall, err = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        o_ref, kv_ref = oracle.recurrent(q, k, v, cu, want_o=True, want_state=not one_doc or Ts == T)
        wall += time.perf_counter() - t0
        if err is None:
            g = w["gpu_o"][:Ts]
            g = (g.float() if g.dtype.is_floating_point and g.element_size() == 2 else g).cpu().numpy()
            e_o = error_vs_oracle(g, o_ref)
            err = {"o_rel_l2": e_o[0], "o_max_abs_rel": e_o[1], "compared": f"o of tokens [0, {Ts}), all heads"}
            if kv_ref is not None:
                e_kv = error_vs_oracle(w["gpu_kv"].cpu().numpy(), kv_ref)
                err.update(kv_state_rel_l2=e_kv[0], kv_state_max_abs_rel=e_kv[1])
        del o_ref, kv_ref
        reps += 1
        threads = oracle.last_threads()
        if wall * threads >= target_cpu_s or reps >= 50:
            break
    th = Ts * H * reps / wall
    hq = max(1, H // 4)
    Ts1 = min(Ts, 32768)
    cu1 = np.array([0, Ts1], dtype=np.int32) if one_doc else cu
    t0 = time.perf_counter()
    oracle.recurrent(q[:Ts1] if one_doc else q, k[:Ts1] if one_doc else k, v[:Ts1] if one_doc else v, cu1,
                     want_o=True, want_state=True, heads=(0, hq), nthreads=1)
    one = (Ts1 if one_doc else Ts) * hq / (time.perf_counter() - t0)
    return {"value": th, "unit": "token·heads/s", "cores": threads, "kind": "oracle",
            "sample": f"first {Ts} tokens x {H} heads of {w['name']} (d={w['d']}), fp64 recurrent form, "
                      f"{reps} repetition(s), {wall:.2f} s wall on {threads} threads",
            "single_thread_value": one, "cpu_model": cpu_model(), "error_vs_oracle": err}


def decode_cpu_baseline(S_sample, steps: int = 200) -> dict:
    """The fp64 oracle's decode step on a sample of the decode workload: the
    incoming states of its first sequences (S_sample, fp32 [pairs, d, d])
    over `steps` steps, scaled to whole-workload steps/s."""
    import la_inputs
    import oracle

    cfg = la_inputs.WORKLOADS["decode_256x64"]
    ns, H, d, seed = cfg["num_seqs"], cfg["H"], cfg["d"], cfg["seed"]
    seqs = S_sample.shape[0] // H
    S = np.ascontiguousarray(S_sample[: seqs * H], dtype=np.float64)
    ins = [tuple(x[:seqs] for x in la_inputs.decode_step_inputs(seed, s % cfg["pool"], ns, H, d, "bf16"))
           for s in range(steps)]
    t0 = time.perf_counter()
    for q, k, v in ins:
        oracle.decode_step(q, k, v, S)
    wall = time.perf_counter() - t0
    return {"value": steps * (seqs * H) / (ns * H) / wall, "unit": "steps/s", "cores": oracle.last_threads(),
            "kind": "oracle", "sample": f"{seqs * H} of {ns * H} (sequence, head) pairs x {steps} steps, "
                                        f"{wall:.2f} s wall, scaled to the whole batch"}


# ------------------------------------------------------------ profile passes

def profile_pass(args, la, torch):
    """Short run for rocprofv3 counter passes: a 256 MiB 1-read + 1-write
    stream (la_bench_stream, the calibration kernel: 268,435,456 bytes read
    and written), then a few calls of the workload."""
    import la_inputs

    lib = la.load()
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    st = lib.la_bench_stream(0, ctypes.c_void_p(src.data_ptr()), None, None, ctypes.c_void_p(dst.data_ptr()),
                             256 << 20, 256, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    torch.cuda.synchronize()
    del src, dst
    w = la_inputs.prefill_inputs(args.workload)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(w["q"]), dev(w["k"]), dev(w["v"])
    cu = torch.from_numpy(w["cu"]).cuda()
    if args.profile_backward:
        dout = dev(la_inputs.normal(la_inputs.WORKLOADS[args.workload]["seed"], 8, q.shape, "bf16", 1.0))
        for _ in range(args.steps):
            la.backward(q, k, v, dout, cu, block=args.block or w["block"], want_dkv_in=False)
    else:
        for _ in range(args.steps):
            la.prefill(q, k, v, cu, block=args.block or w["block"])
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": args.workload, "steps": args.steps, "backward": args.profile_backward}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_1m", choices=["long_1m", "varlen_128k", "prefill_8k", "tiny_fp32"])
    ap.add_argument("--block", type=int, default=0)
    ap.add_argument("--seg-len", type=int, default=0)
    ap.add_argument("--slices", type=int, default=0)
    ap.add_argument("--force-scan", action="store_true")
    ap.add_argument("--slots", type=int, default=0, help="tile slots of the block loop: 0 automatic, 2 or 3")
    ap.add_argument("--rotate", type=int, default=8, help="input sets cycled through the timed steps (at most 8 GiB)")
    ap.add_argument("--small-steps", type=int, default=2000, help="timed steps of the 8k workload")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--profile-backward", action="store_true", help="with --profile-pass: backward calls")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path, so only --gpus 1 is valid",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import causal_linear_attention_la_amd as la

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    la.load()
    if args.profile_pass:
        profile_pass(args, la, torch)
        return
    hip = Hip()
    ceil = stream_ceilings(la, torch, hip)
    prefill_ceiling = ceil["stream_3r1w"]["GBs"]

    small = args.workload in ("prefill_8k", "tiny_fp32")
    steps = args.small_steps if small and args.steps == 20 else args.steps
    head, w = bench_prefill(args.workload, args, la, torch, hip, steps, args.warmup,
                            graph=small and not args.no_graph, keep_sets=True)
    with_ceiling(head["roofline"], prefill_ceiling)
    head["whole_call"]["frac_of_measured_ceiling"] = head["whole_call"]["achieved"] / prefill_ceiling
    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "whole_call": head["whole_call"],
        "gpu_ms_per_step": head["gpu_ms_per_step"],
        "ceilings": ceil,
    }
    if args.workload == "long_1m" and not args.no_extra and not args.block:
        rec["long_1m_block128"] = bench_block(la, torch, hip, w, 128, 3)
    if not args.no_extra and not args.block and w["dtype"] == "bf16":
        rec["decay"] = bench_decay(la, torch, hip, w, max(3, args.steps // 2))
    if not args.no_backward:
        rec["backward"] = bench_backward(args, la, torch, hip, w, w.pop("dev_sets"), max(2, args.steps // 4))
        with_ceiling(rec["backward"]["roofline"], prefill_ceiling)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    else:
        rec["cpu_baseline"] = None
    w.pop("dev_sets", None)
    del w
    torch.cuda.empty_cache()

    if not args.no_extra:
        extras = {}
        for name in ("varlen_128k", "long_1m", "prefill_8k"):
            if name == args.workload:
                continue
            sm = name == "prefill_8k"
            r, wx = bench_prefill(name, args, la, torch, hip, args.small_steps if sm else args.steps, args.warmup,
                                  graph=sm and not args.no_graph, keep_sets=name == "varlen_128k")
            with_ceiling(r["roofline"], prefill_ceiling)
            r["whole_call"]["frac_of_measured_ceiling"] = r["whole_call"]["achieved"] / prefill_ceiling
            if name == "varlen_128k" and not args.block:
                r["block128"] = bench_block(la, torch, hip, wx, 128, 3)
            extras[name] = r
            wx.pop("dev_sets", None)
            del wx
            torch.cuda.empty_cache()
        rec["workloads"] = extras
    if not args.no_decode:
        rec["decode"] = bench_decode(args, la, torch, hip)
        with_ceiling(rec["decode"]["roofline"], ceil["copy_1r1w"]["GBs"])
        if not args.no_cpu_baseline:
            rec["decode"]["cpu_baseline"] = decode_cpu_baseline(DECODE_SAMPLE["S"])
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
