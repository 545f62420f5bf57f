#!/usr/bin/env python3
"""Benchmark: causal linear attention (Lightning-style) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_8k]

A step is one pass of the hot path over one batch of synthetic input: one
la_prefill call over the workload (segment states, prefix scan when needed,
block loop).  The default workload is the 8-head x 8192-token bf16 prefill
(d = 128, block 64).  Inputs are generated on the host from fixed seeds,
copied to HBM before timing, and rotated over several input sets so that the
timed steps read HBM rather than the 256 MB last-level cache.  The decode
workload (256 sequences x 64 heads, fp32 state, 1000 steps) is timed in the
same run and reported under "decode", and the prefill's backward
(la_prefill_backward: dq, dk, dv) over the same workload under "backward", with
a forward + backward pair sharing the forward's workspace under
"backward"/"train_step".

Prints one JSON line.  `roofline` is for the block-loop kernel: algorithmic
bytes (q, k, v read + o written, 8 d bytes per token-head) per launch over its
average duration, measured with HIP events stamped on the launch stream
around every 8th launch inside the timed region (--event-stride; stamping
every launch costs several microseconds per step).  `cpu_baseline` times the fp64
oracle (the recurrent form) on the host cores for the same workload.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0

KERNEL_SOURCES = ["la_prefill_kernels.h", "la_prefill_v2.h", "la_device.h", "la_tiles.h", "la_prefill_launch.inl",
                  "la_prefill_bf16.hip", "la_host.cpp"]
MAIN_KERNEL = {1: "la_prefill_main_kernel", 2: "la_prefill_main_v2"}  # by the plan's block-loop variant
DECODE_SOURCES = ["la_decode_kernels.h", "la_device.h"]


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


def cpu_baseline(w, target_cpu_s: float = 10.0) -> dict:
    """The fp64 oracle as it stands, over the whole workload, repeated until
    about target_cpu_s seconds of CPU time have been spent."""
    import oracle

    oracle.build()
    reps, wall = 0, 0.0
    while True:
        t0 = time.perf_counter()
        o_ref, kv_ref = oracle.recurrent(w["q"], w["k"], w["v"], w["cu"], want_o=True, want_state=True)
        wall += time.perf_counter() - t0
        if reps == 0 and "gpu_o" in w:
            w["error_vs_oracle"] = error_vs_oracle(w, o_ref, kv_ref)
        del o_ref, kv_ref
        reps += 1
        threads = oracle.last_threads()
        if wall * threads >= target_cpu_s or reps >= 50:
            break
    th = w["T"] * w["H"] * reps / wall
    # one thread on a quarter of the heads, for a per-core figure
    hq = max(1, w["H"] // 4)
    t0 = time.perf_counter()
    oracle.recurrent(w["q"], w["k"], w["v"], w["cu"], want_o=True, want_state=True, heads=(0, hq), nthreads=1)
    one = w["T"] * hq / (time.perf_counter() - t0)
    return {"value": th, "unit": "token·heads/s", "cores": threads, "kind": "oracle",
            "sample": f"whole {w['name']} workload ({w['T']} tokens x {w['H']} heads, d={w['d']}), "
                      f"fp64 recurrent form, {reps} repetitions, {wall:.2f} s wall",
            "single_thread_value": one, "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_bandwidth(torch, hip, nbytes: int = 1 << 30, reps: int = 20) -> float:
    """Measured device copy bandwidth (GB/s, read + write bytes) of a 1 GiB
    device-to-device copy: a second, practical roofline beside the datasheet's."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(e0, stream)
    for _ in range(reps):
        dst.copy_(src)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    s = hip.elapsed_ms(e0, e1) / 1e3
    hip.destroy(e0)
    hip.destroy(e1)
    del src, dst
    return 2 * nbytes * reps / s / 1e9


def bench_prefill(args, la, torch, hip):
    import la_inputs

    name = args.workload
    cfg = la_inputs.WORKLOADS[name]
    w = la_inputs.prefill_inputs(name)
    w["name"] = name
    T, H, d, block = w["T"], w["H"], w["d"], args.block or w["block"]
    dt = la.LA_BF16 if w["dtype"] == "bf16" else la.LA_FP32
    num_seqs = len(w["cu"]) - 1
    opts = dict(seg_len=args.seg_len, value_slices=args.slices, force_scan=args.force_scan, slots=args.slots)
    plan = la.la_prefill_plan(T, num_seqs, H, d, block, dt, la.make_opts(**opts))

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    # input sets: set 0 is the seeded workload, the others are copies shifted
    # by one token per set (same statistics, different bytes in HBM)
    per_set = 4 * T * H * d * (2 if w["dtype"] == "bf16" else 4)
    nsets = max(1, min(args.rotate, int((8 << 30) // max(per_set, 1))))
    q0, k0, v0 = dev(w["q"]), dev(w["k"]), dev(w["v"])
    sets = []
    for i in range(nsets):
        sh = i % max(T, 1)
        q, k, v = (torch.roll(x, sh, 0).contiguous() if sh else x for x in (q0, k0, v0))
        sets.append((q, k, v, torch.empty_like(q)))
    w["dev_sets"] = sets
    cu = torch.from_numpy(w["cu"]).cuda()
    kv = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device="cuda")
    ws_bytes = plan["workspace_bytes"]
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i, ev0=None, ev1=None):
        q, k, v, o = sets[i % nsets]
        la.prefill(q, k, v, cu, block=block, out=o, kv_state_out=kv, workspace=ws, begin_event=ev0, end_event=ev1,
                   **opts)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    # The block-loop kernel of every event_stride-th step in the timed region
    # is launched with start/end events (hipExtLaunchKernel); stamping every
    # launch would itself cost several microseconds per step.
    # (short timed regions -- long steps -- stamp every launch: there the cost is noise)
    stride = max(1, args.event_stride) if args.event_stride else (8 if args.steps >= 128 else 1)
    evs = {i: (hip.event(), hip.event()) for i in range(0, K, stride)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if i in evs:
            step(i, evs[i][0], evs[i][1])
        else:
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = [hip.elapsed_ms(a, b) for a, b in evs.values()]
    for a, b in evs.values():
        hip.destroy(a)
        hip.destroy(b)

    # the same steps replayed from a HIP graph (launch overhead removed)
    graph_value = None
    if not args.no_graph:
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
        reps = max(1, K // nsets)
        g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        graph_elapsed = time.perf_counter() - t1
        graph_value = T * H * nsets * reps / graph_elapsed

    avg_kernel_s = float(np.mean(kernel_ms)) / 1e3
    algo_bytes = T * H * 8 * d * (1 if w["dtype"] == "bf16" else 2)
    achieved = algo_bytes / avg_kernel_s / 1e9
    sha = sources_sha(KERNEL_SOURCES)
    kname = MAIN_KERNEL[plan["variant"]]
    traffic = load_traffic(kname, name, sha)
    value = T * H * K / elapsed
    roof_th = HBM_PEAK_GBS * 1e9 / (algo_bytes / (T * H))  # whole step at HBM peak
    rec = {
        "metric": "prefill tokens·heads/s (bf16, d=128) + % roofline; decode steps/s",
        "value": value,
        "unit": "token·heads/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": name, "documents": num_seqs, "heads": H, "tokens": T, "head_dim": d, "block": block,
                   "seg_len": plan["seg_len"], "value_slices": plan["value_slices"],
                   "segments": plan["num_segments"], "scan": plan["scan"], "slots": plan["slots"],
                   "workgroups": plan["units"], "event_stride": stride,
                   "input_sets": nsets},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel_ms": avg_kernel_s * 1e3,
                     "algorithmic_bytes": algo_bytes, "kernel_sources_sha": sha},
        "path_roofline": {"token_heads_per_s": roof_th, "frac": value / roof_th},
        "graph_replay_value": graph_value,
    }
    if not args.no_cpu_baseline:
        # outputs of the seeded input set, for the error against the oracle
        step(0)
        torch.cuda.synchronize()
        o0 = sets[0][3]
        w["gpu_o"] = (o0.float() if o0.dtype == torch.bfloat16 else o0).cpu().numpy()
        w["gpu_kv"] = kv.cpu().numpy()
    return rec, w


def error_vs_oracle(w, o_ref, kv_ref) -> dict:
    """rel-L2 and max-abs error (relative to max |ref|) of the GPU outputs
    of the seeded input set against the fp64 oracle."""
    def errs(g, r):
        g = np.asarray(g, dtype=np.float64).ravel()
        r = np.asarray(r, dtype=np.float64).ravel()
        den = max(float(np.linalg.norm(r)), 1e-300)
        return float(np.linalg.norm(g - r) / den), float(np.max(np.abs(g - r)) / max(float(np.max(np.abs(r))), 1e-300))
    o_l2, o_max = errs(w["gpu_o"], o_ref)
    kv_l2, kv_max = errs(w["gpu_kv"], kv_ref)
    return {"o_rel_l2": o_l2, "o_max_abs_rel": o_max, "kv_state_rel_l2": kv_l2, "kv_state_max_abs_rel": kv_max}


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
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(e0, stream)
    for i in range(steps):
        la.decode(*sets[i % pool], S, out=o)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = hip.elapsed_ms(e0, e1) / 1e3
    hip.destroy(e0)
    hip.destroy(e1)
    bytes_step = ns * H * (2 * d * d * 4 + 4 * d * 2)
    achieved = bytes_step * steps / gpu_s / 1e9
    return {"workload": "decode_256x64", "value": steps / wall, "unit": "steps/s", "steps": steps,
            "ms_per_step": wall / steps * 1e3, "gpu_ms_per_step": gpu_s / steps * 1e3,
            "roofline": {"bound": "hbm", "kernel": "la_decode_kernel", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "bytes_per_step": bytes_step,
                         "kernel_sources_sha": sources_sha(DECODE_SOURCES)}}


def bench_backward(args, la, torch, hip, w, dev_sets):
    """la_prefill_backward over the same workload: dq, dk, dv from dO with no
    incoming state and no final-state gradient.  Algorithmic bytes per call:
    q, k, v, dO read and dq, dk, dv written once, 14 d bytes per token-head
    in bf16.  Timed with HIP events on the launch stream around all calls."""
    import la_inputs

    T, H, d = w["T"], w["H"], w["d"]
    esz = 2 if w["dtype"] == "bf16" else 4
    block = args.block or w["block"]
    opts = dict(seg_len=args.seg_len, value_slices=args.slices, force_scan=args.force_scan, slots=args.slots)
    cu = torch.from_numpy(w["cu"]).cuda()
    d0 = la_inputs.normal(la_inputs.WORKLOADS[w["name"]]["seed"], 8, (T, H, d), w["dtype"], 1.0)
    dout0 = torch.from_numpy(d0.view(np.int16)).view(torch.bfloat16).cuda() if d0.dtype == np.uint16 \
        else torch.from_numpy(d0).cuda()
    sets = []
    for i, (q, k, v, _) in enumerate(dev_sets):
        dout = torch.roll(dout0, i, 0).contiguous() if i else dout0
        sets.append((q, k, v, dout))
    outs = (torch.empty_like(dout0), torch.empty_like(dout0), torch.empty_like(dout0), None)
    num_seqs = len(w["cu"]) - 1
    dt = la.LA_BF16 if w["dtype"] == "bf16" else la.LA_FP32
    need = la.la_prefill_workspace_size_ex(T, num_seqs, H, d, block, dt, la.make_opts(**opts))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")

    def call(i):
        q, k, v, dout = sets[i % len(sets)]
        la.backward(q, k, v, dout, cu, block=block, want_dkv_in=False, workspace=ws, out=outs, **opts)

    for i in range(max(1, args.warmup // 4)):
        call(i)
    torch.cuda.synchronize()
    K = max(1, args.steps // 4)
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(e0, stream)
    for i in range(K):
        call(i)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = hip.elapsed_ms(e0, e1) / 1e3
    hip.destroy(e0)
    hip.destroy(e1)
    algo = T * H * 14 * d * esz // 2
    achieved = algo * K / gpu_s / 1e9
    rec = {"workload": w["name"], "value": T * H * K / wall, "unit": "token·heads/s", "steps": K,
           "ms_per_step": wall / K * 1e3, "gpu_ms_per_step": gpu_s / K * 1e3,
           "roofline": {"bound": "hbm", "kernel": "la_prefill_backward (3 prefill passes)", "achieved": achieved,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                        "algorithmic_bytes": algo}}

    # One training step's attention work: the forward, then the backward handed
    # the forward's workspace (its dq pass reuses the forward's segment states).
    fo = torch.empty_like(dout0)
    fkv = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device="cuda")

    def train(i):
        q, k, v, dout = sets[i % len(sets)]
        la.prefill(q, k, v, cu, block=block, out=fo, kv_state_out=fkv, workspace=ws, **opts)
        la.backward(q, k, v, dout, cu, block=block, want_dkv_in=False, out=outs, forward_workspace=ws, **opts)

    for i in range(max(1, args.warmup // 4)):
        train(i)
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(e0, stream)
    for i in range(K):
        train(i)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    tr_s = hip.elapsed_ms(e0, e1) / 1e3
    hip.destroy(e0)
    hip.destroy(e1)
    talgo = T * H * 22 * d * esz // 2  # forward 8d + backward 14d bytes per token-head
    tach = talgo * K / tr_s / 1e9
    rec["train_step"] = {"value": T * H * K / tr_s, "unit": "token·heads/s", "gpu_ms_per_step": tr_s / K * 1e3,
                         "roofline": {"bound": "hbm", "achieved": tach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": tach / HBM_PEAK_GBS, "algorithmic_bytes": talgo}}
    return rec


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


def profile_pass(args, la, torch):
    """Short run for rocprofv3 counter passes: a 256 MiB device copy (the
    calibration kernel) then a few prefill steps of the workload."""
    import la_inputs

    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
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
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill_8k",
                    choices=["prefill_8k", "varlen_128k", "long_1m", "tiny_fp32"])
    ap.add_argument("--block", type=int, default=0)
    ap.add_argument("--seg-len", type=int, default=0)
    ap.add_argument("--slices", type=int, default=0)
    ap.add_argument("--force-scan", action="store_true")
    ap.add_argument("--slots", type=int, default=0, help="tile slots of the block loop: 0 automatic, 2 or 3")
    ap.add_argument("--rotate", type=int, default=8, help="input sets cycled through the timed steps")
    ap.add_argument("--event-stride", type=int, default=0,
                    help="stamp the block-loop kernel of every n-th timed step with events "
                         "(0: every 8th with 128 or more steps, else every one)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--profile-backward", action="store_true", help="with --profile-pass: backward calls")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
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
    rec, w = bench_prefill(args, la, torch, hip)
    if not args.no_backward:
        rec["backward"] = bench_backward(args, la, torch, hip, w, w.pop("dev_sets"))
    else:
        w.pop("dev_sets")
    if not args.no_decode:
        rec["decode"] = bench_decode(args, la, torch, hip)
    copy = copy_bandwidth(torch, hip)
    for part in (rec, rec.get("backward"), rec.get("decode")):
        if part:
            part["roofline"]["measured_copy_GBs"] = copy
            part["roofline"]["frac_of_measured_copy"] = part["roofline"]["achieved"] / copy
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
        rec["error_vs_oracle"] = w.get("error_vs_oracle")
        if "decode" in rec:
            rec["decode"]["cpu_baseline"] = decode_cpu_baseline(DECODE_SAMPLE["S"])
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
