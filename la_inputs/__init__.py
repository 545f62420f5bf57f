"""Seeded synthetic inputs for the causal linear attention workloads.

Shared by the GPU path's tests and benchmark and by the oracle's tests.  It
draws random inputs only (see ``gen.c``) and holds none of the attention
arithmetic.  Every array is a deterministic function of (seed, tensor id,
element index), so the same bytes reach both sides.

Workloads (sizes of the MiniMax-01 Lightning Attention layers: 64 heads of
width 128, contexts up to 1M tokens, packed documents, prefill and decode):

* ``tiny_fp32``    2 heads x 256 tokens, d=16, fp32, block 32
* ``prefill_8k``   8 heads x 8192 tokens, d=128, bf16, block 64
* ``varlen_128k``  64 heads, 131072 packed tokens, documents log-uniform in
  [512, 32768] (last one cut to fit), d=128, bf16, block 64
* ``long_1m``      8 heads x 1,048,576 tokens, d=128, bf16, block 64 or 128
* ``decode_256x64`` 256 sequences x 64 heads, d=128, bf16 tokens, fp32 state
  whose prefix length is log-uniform in [1024, 1048576) per sequence

q, k, v entries are i.i.d. N(0, 1/d), rounded to fp32 then (for bf16) to
bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_lagen.so")
_SRC = os.path.join(_HERE, "gen.c")

# tensor ids inside one workload seed
TID_Q, TID_K, TID_V, TID_DOCS, TID_STATE, TID_PREFIX = 0, 1, 2, 3, 4, 5
TID_STEP0 = 16  # decode step-set s uses ids 16 + 3 s + {0, 1, 2}

WORKLOADS = {
    "tiny_fp32": dict(kind="prefill", seed=101, T=256, H=2, d=16, block=32, dtype="fp32", docs=None),
    "prefill_8k": dict(kind="prefill", seed=102, T=8192, H=8, d=128, block=64, dtype="bf16", docs=None),
    "varlen_128k": dict(kind="prefill", seed=103, T=131072, H=64, d=128, block=64, dtype="bf16",
                        docs=(512, 32768)),
    "long_1m": dict(kind="prefill", seed=104, T=1048576, H=8, d=128, block=64, dtype="bf16", docs=None),
    "decode_256x64": dict(kind="decode", seed=105, num_seqs=256, H=64, d=128, dtype="bf16",
                          prefix=(1024, 1048576), steps=1000, pool=64),
}


def build(force: bool = False) -> str:
    """Compile gen.c with gcc into _lagen.so (in place)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        vp = ctypes.c_void_p
        lib.lagen_stream_key.argtypes = [u64, u64]
        lib.lagen_stream_key.restype = u64
        lib.lagen_normal_bf16.argtypes = [u64, u64, dbl, u64, i64, vp, ctypes.c_int]
        lib.lagen_normal_f32.argtypes = [u64, u64, dbl, u64, i64, vp, ctypes.c_int]
        lib.lagen_ternary.argtypes = [u64, u64, i64, vp, ctypes.c_int, ctypes.c_int]
        lib.lagen_doc_lengths.argtypes = [u64, u64, i64, i64, i64, vp, i32]
        lib.lagen_doc_lengths.restype = i32
        lib.lagen_prefix_len.argtypes = [u64, u64, i64, i64, i64]
        lib.lagen_prefix_len.restype = i64
        lib.lagen_decode_states.argtypes = [u64, u64, u64, i64, i64, i64, i64, i64, vp, vp, ctypes.c_int]
        lib.lagen_decode_states.restype = ctypes.c_int
        lib.lagen_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.lagen_f32_to_bf16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def normal(seed: int, tensor_id: int, shape, dtype: str, scale: float = 1.0, offset: int = 0,
           nthreads: int = 0) -> np.ndarray:
    """N(0,1)*scale; dtype 'bf16' returns uint16 bit patterns, 'fp32' float32."""
    n = int(np.prod(shape))
    lib = _load()
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.lagen_normal_bf16(seed, tensor_id, scale, offset, n, _ptr(out), nthreads)
    elif dtype == "fp32":
        out = np.empty(n, dtype=np.float32)
        lib.lagen_normal_f32(seed, tensor_id, scale, offset, n, _ptr(out), nthreads)
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def ternary(seed: int, tensor_id: int, shape, dtype: str, nthreads: int = 0) -> np.ndarray:
    """Entries uniform in {-1, 0, 1} (exact in bf16 and fp32)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    _load().lagen_ternary(seed, tensor_id, n, _ptr(out), 0 if dtype == "bf16" else 1, nthreads)
    return out.reshape(shape)


def doc_lengths(seed: int, total: int, lo: int, hi: int, tensor_id: int = TID_DOCS) -> np.ndarray:
    """cu_seqlens (int32) of documents with length floor(exp(U[ln lo, ln hi))), last cut to fit."""
    cap = int(total // max(1, lo)) + 2 if lo > 0 else total + 2
    cap = max(cap, 2)
    cu = np.zeros(cap + 1, dtype=np.int32)
    nd = _load().lagen_doc_lengths(seed, tensor_id, total, lo, hi, _ptr(cu), cap)
    if nd < 0:
        raise RuntimeError("document capacity exceeded")
    return cu[: nd + 1].copy()


def prefix_lengths(seed: int, num_seqs: int, lo: int, hi: int, tensor_id: int = TID_PREFIX) -> np.ndarray:
    lib = _load()
    return np.array([lib.lagen_prefix_len(seed, tensor_id, s, lo, hi) for s in range(num_seqs)], dtype=np.int64)


def decode_states(seed: int, num_seqs: int, H: int, d: int, lo: int, hi: int, fixed_n=None,
                  nthreads: int = 0) -> np.ndarray:
    """fp32 [num_seqs*H, d, d] incoming states distributed as K^T V over a prefix of
    n ~ floor(exp(U[ln lo, ln hi))) tokens (one n per sequence) of N(0, I/d) rows."""
    out = np.empty((num_seqs * H, d, d), dtype=np.float32)
    fn = None
    if fixed_n is not None:
        fn = np.ascontiguousarray(np.asarray(fixed_n, dtype=np.int64).reshape(-1))
        assert fn.size == num_seqs * H
    rc = _load().lagen_decode_states(seed, TID_STATE, TID_PREFIX, num_seqs, H, d, lo, hi,
                                     _ptr(fn) if fn is not None else None, _ptr(out), nthreads)
    if rc == -2:
        raise ValueError("prefix lengths must be >= d")
    if rc != 0:
        raise ValueError("unsupported d")
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def prefill_inputs(name_or_cfg, T: int | None = None, nthreads: int = 0) -> dict:
    """q, k, v ([T, H, d]; uint16 bf16 bits or float32) and cu_seqlens for a prefill
    workload.  ``T`` truncates the token count (same per-element values as the
    full workload for the first T tokens when there is one document)."""
    cfg = dict(WORKLOADS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    T = cfg["T"] if T is None else T
    H, d, seed, dt = cfg["H"], cfg["d"], cfg["seed"], cfg["dtype"]
    scale = 1.0 / np.sqrt(d)
    q = normal(seed, TID_Q, (T, H, d), dt, scale, nthreads=nthreads)
    k = normal(seed, TID_K, (T, H, d), dt, scale, nthreads=nthreads)
    v = normal(seed, TID_V, (T, H, d), dt, scale, nthreads=nthreads)
    if cfg.get("docs"):
        lo, hi = cfg["docs"]
        cu = doc_lengths(seed, T, lo, hi)
    else:
        cu = np.array([0, T], dtype=np.int32)
    return dict(q=q, k=k, v=v, cu=cu, H=H, d=d, T=T, dtype=dt, block=cfg.get("block", 64))


def decode_step_inputs(seed: int, step_set: int, num_seqs: int, H: int, d: int, dtype: str,
                       nthreads: int = 0) -> tuple:
    """q, k, v [num_seqs, H, d] of one decode step set."""
    scale = 1.0 / np.sqrt(d)
    base = TID_STEP0 + 3 * step_set
    return tuple(normal(seed, base + i, (num_seqs, H, d), dtype, scale, nthreads=nthreads) for i in range(3))
