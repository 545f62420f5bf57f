"""C-ABI checks that need no GPU: the library loads, exports every entry point
the headers in include/ declare, and rejects bad arguments on the host before
anything is enqueued (only invalid calls are made here)."""
import ast
import glob
import ctypes
import os
import re
import subprocess

import pytest

import causal_linear_attention_la_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(la.LIB_PATH):
        la.build()
    return la.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(?:la_status|size_t|const char\s*\*)\s+(la_\w+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(la.EXPORTED) == set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (la_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)


def test_status_strings(lib):
    assert la.status_string(0) == "LA_OK"
    assert la.status_string(3) == "LA_ERR_WORKSPACE"
    assert la.status_string(99) == "LA_ERR_UNKNOWN"


G = 1 << 40  # fake device addresses: validation rejects before any use


def _prefill(**kw):
    a = dict(q=G, k=2 * G, v=3 * G, o=4 * G, cu=5 * G, H=8, d=128, block=64, kv=6 * G, num_seqs=1, T=8192,
             dtype=la.LA_BF16, ws=7 * G, ws_bytes=1 << 30)
    a.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    return la.la_prefill(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), vp(a["cu"]), a["H"], a["d"], a["block"],
                         vp(a["kv"]), a["num_seqs"], a["T"], a["dtype"], vp(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), la.LA_ERR_INVALID_ARG),
    (dict(o=0), la.LA_ERR_INVALID_ARG),
    (dict(cu=0), la.LA_ERR_INVALID_ARG),
    (dict(H=0), la.LA_ERR_INVALID_ARG),
    (dict(num_seqs=0), la.LA_ERR_INVALID_ARG),
    (dict(T=-5), la.LA_ERR_INVALID_ARG),
    (dict(d=48), la.LA_ERR_UNSUPPORTED),
    (dict(block=16), la.LA_ERR_UNSUPPORTED),
    (dict(dtype=9), la.LA_ERR_UNSUPPORTED),
    (dict(dtype=la.LA_FP32, block=128), la.LA_ERR_UNSUPPORTED),
    (dict(q=G + 8), la.LA_ERR_INVALID_ARG),
    (dict(o=G + 4096), la.LA_ERR_INVALID_ARG),       # o overlaps q
    (dict(kv=3 * G + 16), la.LA_ERR_INVALID_ARG),    # state overlaps v
    (dict(kv=6 * G + 4), la.LA_ERR_INVALID_ARG),     # misaligned state
    (dict(ws=0), la.LA_ERR_WORKSPACE),
    (dict(ws_bytes=16), la.LA_ERR_WORKSPACE),
    (dict(ws=7 * G + 64), la.LA_ERR_INVALID_ARG),    # workspace not 256-aligned
])
def test_prefill_rejects(lib, kw, status):
    assert _prefill(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), la.LA_ERR_INVALID_ARG),
    (dict(S=0), la.LA_ERR_INVALID_ARG),
    (dict(num_seqs=0), la.LA_ERR_INVALID_ARG),
    (dict(H=-1), la.LA_ERR_INVALID_ARG),
    (dict(d=100), la.LA_ERR_UNSUPPORTED),
    (dict(dtype=3), la.LA_ERR_UNSUPPORTED),
    (dict(o=G), la.LA_ERR_INVALID_ARG),
    (dict(S=G + 16), la.LA_ERR_INVALID_ARG),
    (dict(S=6 * G + 8), la.LA_ERR_INVALID_ARG),
])
def test_decode_rejects(lib, kw, status):
    a = dict(q=G, k=2 * G, v=3 * G, S=6 * G, o=4 * G, num_seqs=256, H=64, d=128, dtype=la.LA_BF16)
    a.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x else None
    assert la.la_decode(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["S"]), vp(a["o"]), a["num_seqs"], a["H"], a["d"],
                        a["dtype"], None) == status


@pytest.mark.parametrize("args", [
    (3, G, 0, 0, 4 * G, 1 << 20, 256, 0),       # unknown mode
    (0, 0, 0, 0, 4 * G, 1 << 20, 256, 0),       # no source
    (1, G, 0, 3 * G, 4 * G, 1 << 20, 256, 0),   # three-source mode with a missing source
    (0, G, 0, 0, 0, 1 << 20, 256, 0),           # no destination
    (0, G + 8, 0, 0, 4 * G, 1 << 20, 256, 0),   # misaligned source
    (0, G, 0, 0, 4 * G, 100, 256, 0),           # size not a multiple of 16
    (0, G, 0, 0, 4 * G, 1 << 20, 0, 0),         # no workgroups
])
def test_bench_stream_rejects(lib, args):
    mode, a, b, c, dst, n, wgs, nt = args
    vp = lambda x: ctypes.c_void_p(x) if x else None
    assert la.la_bench_stream(mode, vp(a), vp(b), vp(c), vp(dst), n, wgs, nt, None) == la.LA_ERR_INVALID_ARG


def test_decay_entry_points_reject(lib):
    """The decayed prefill and decode refuse a missing, misaligned or
    overlapping factor array on the host, and otherwise validate as the plain calls."""
    vp = ctypes.c_void_p

    def pre(decay, o=4 * G, kv=6 * G, d=128):
        return la.la_prefill_decay(vp(G), vp(2 * G), vp(3 * G), vp(o), vp(5 * G), 8, d, 64, vp(decay) if decay else None,
                                   None, vp(kv), 1, 8192, la.LA_BF16, vp(7 * G), 1 << 30, None, None)

    assert pre(0) == la.LA_ERR_INVALID_ARG
    assert pre(9 * G + 2) == la.LA_ERR_INVALID_ARG            # misaligned
    assert pre(4 * G + 64) == la.LA_ERR_INVALID_ARG           # inside o
    assert pre(6 * G + 64) == la.LA_ERR_INVALID_ARG           # inside the final states
    assert pre(7 * G + 512) == la.LA_ERR_INVALID_ARG          # inside the workspace
    assert pre(9 * G, d=48) == la.LA_ERR_UNSUPPORTED          # the plain call's checks follow

    def dec(decay, S=6 * G, o=4 * G):
        return la.la_decode_decay(vp(G), vp(2 * G), vp(3 * G), vp(decay) if decay else None, vp(S), vp(o), 256, 64,
                                  128, la.LA_BF16, None)

    assert dec(0) == la.LA_ERR_INVALID_ARG
    assert dec(9 * G + 1) == la.LA_ERR_INVALID_ARG
    assert dec(6 * G + 4096) == la.LA_ERR_INVALID_ARG         # inside the state
    assert dec(4 * G + 16) == la.LA_ERR_INVALID_ARG           # inside o


def test_noalloc_refuses_plans_beyond_its_array(lib):
    """la_prefill_noalloc refuses, on the host and before any device call, a
    plan whose workspace exceeds the library's static 32 MiB array."""
    T, H, d, B = 353, 274, 128, 32  # two segments of 352 tokens x 274 heads of 64 KiB states
    assert la.la_prefill_plan(T, 1, H, d, B, la.LA_BF16)["workspace_bytes"] > 32 << 20
    vp = ctypes.c_void_p
    st = la.la_prefill_noalloc(vp(G), vp(2 * G), vp(3 * G), vp(4 * G), vp(5 * G), H, d, B, vp(6 * G), 1, T,
                               la.LA_BF16, None)
    assert st == la.LA_ERR_WORKSPACE
    # shape errors come first, as in la_prefill
    assert la.la_prefill_noalloc(vp(G), vp(2 * G), vp(3 * G), vp(4 * G), vp(5 * G), 8, 48, 64, None, 1, 8192,
                                 la.LA_BF16, None) == la.LA_ERR_UNSUPPORTED


def test_plans(lib):
    p = la.la_prefill_plan(8192, 1, 8, 128, 64, la.LA_BF16)
    assert p["units"] == p["num_segments"] * 8 * p["value_slices"] and p["seg_len"] % 64 == 0
    assert p["workspace_bytes"] == la.la_prefill_workspace_size(8192, 1, 8, 128, 64, la.LA_BF16)
    p = la.la_prefill_plan(256, 1, 2, 16, 32, la.LA_FP32)
    assert p["num_segments"] == 1 and p["workspace_bytes"] == 0
    p = la.la_prefill_plan(1048576, 1, 8, 128, 64, la.LA_BF16)
    assert p["units"] >= 256
    o = la.make_opts(seg_len=64, value_slices=2)
    p = la.la_prefill_plan(8192, 1, 8, 128, 64, la.LA_BF16, o)
    assert (p["seg_len"], p["value_slices"], p["num_segments"], p["scan"]) == (64, 2, 128, 1)
    assert p["workspace_bytes"] >= 128 * 8 * 128 * 128 * 4
    with pytest.raises(la.LAError):
        la.la_prefill_plan(8192, 1, 8, 128, 64, la.LA_BF16, la.make_opts(seg_len=100))
    # document pieces on the packed 131072-token workload (20 documents, 64 heads): at most 24 pieces
    p = la.la_prefill_plan(131072, 20, 64, 128, 64, la.LA_BF16)
    assert p["packed"] == 1 and p["units"] == 24 * 64 and p["scan"] == 0
    assert la.la_prefill_plan(8192, 1, 8, 128, 64, la.LA_BF16)["packed"] == 0
    assert la.la_prefill_plan(131072, 20, 64, 128, 64, la.LA_BF16, la.make_opts(work_list=1))["packed"] == 0
    with pytest.raises(la.LAError):  # a document could need more than 16 earlier pieces
        la.la_prefill_plan(8192, 2, 8, 128, 64, la.LA_BF16, la.make_opts(seg_len=64, work_list=2))
    # tile slots of the transpose-read loop: three on long segments, two on short ones
    assert la.la_prefill_plan(8192, 1, 8, 128, 64, la.LA_BF16)["slots"] == 2
    assert la.la_prefill_plan(1048576, 1, 8, 128, 64, la.LA_BF16)["slots"] == 3
    assert la.la_prefill_plan(8192, 1, 8, 128, 64, la.LA_BF16, la.make_opts(slots=3))["slots"] == 3
    with pytest.raises(la.LAError):
        la.la_prefill_plan(8192, 1, 8, 64, 64, la.LA_BF16, la.make_opts(slots=3))


def test_backward_workspace_size(lib):
    """The backward's workspace with room for the transposed segment states:
    the forward's bytes (rounded to 256) plus one fp32 d x d state per segment
    state and head, also rounded; the forward's size when the plan keeps no
    segment states or runs the generic loop; 0 for shapes the planner rejects."""
    r256 = lambda x: (x + 255) // 256 * 256
    for T, D, H, d, B, dt, o in [(8192, 1, 8, 128, 64, la.LA_BF16, None),
                                 (1048576, 1, 8, 128, 64, la.LA_BF16, None),
                                 (8192, 1, 8, 128, 64, la.LA_BF16, la.make_opts(seg_len=64, value_slices=2)),
                                 (131072, 20, 64, 128, 64, la.LA_BF16, la.make_opts(seg_len=8192, work_list=2))]:
        p = la.la_prefill_plan(T, D, H, d, B, dt, o)
        states = (T // p["seg_len"]) if p["packed"] else p["num_segments"] - 1
        got = la.la_prefill_backward_workspace_size(T, D, H, d, B, dt, o)
        assert got == r256(p["workspace_bytes"]) + r256(states * H * d * d * 4), (T, D, H, p)
        assert got > la.la_prefill_workspace_size_ex(T, D, H, d, B, dt, o)
    # no segment states (one segment; every document one piece), generic loop: the forward's size
    assert la.la_prefill_backward_workspace_size(256, 1, 2, 16, 32, la.LA_FP32) == 0
    p = la.la_prefill_plan(131072, 20, 64, 128, 64, la.LA_BF16)
    assert la.la_prefill_backward_workspace_size(131072, 20, 64, 128, 64, la.LA_BF16) == \
        r256(p["workspace_bytes"]) + r256((131072 // p["seg_len"]) * 64 * 128 * 128 * 4)
    o = la.make_opts(variant=1, seg_len=512)
    assert la.la_prefill_backward_workspace_size(8192, 1, 8, 128, 64, la.LA_BF16, o) == \
        la.la_prefill_workspace_size_ex(8192, 1, 8, 128, 64, la.LA_BF16, o)
    assert la.la_prefill_backward_workspace_size(8192, 1, 8, 48, 64, la.LA_BF16) == 0


def test_host_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "hvc")
    src = [os.path.join(ROOT, "tests", "native", "host_validation_check.cpp"),
           os.path.join(ROOT, "causal_linear_attention_la_amd", "csrc", "la_host.cpp")]
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", *src, "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_no_undefined_library_symbols(lib):
    """Every kernel launch stub the library calls is defined in it (a missing
    template instantiation would otherwise only show up as a load failure at run time)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", la.LIB_PATH], capture_output=True, text=True).stdout
    missing = [l for l in out.splitlines() if "_ZN2la" in l]
    assert not missing, missing


def test_one_hip_runtime_in_the_process():
    """Loading the library first, then torch, leaves one HIP runtime in the
    process: torch's bundled one, to which the library binds (the binding
    imports torch before it loads the library).  Two runtimes would each see
    the other's tensors and streams as foreign."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import causal_linear_attention_la_amd as la\n"
        "la.load()\n"
        "import torch\n"
        "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))\n" % ROOT
    )
    out = subprocess.run(["python3", "-c", code], capture_output=True, text=True, check=True).stdout.strip()
    paths = ast.literal_eval(out)
    assert len(paths) == 1, paths
