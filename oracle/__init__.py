"""fp64 CPU oracle for causal linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg import this package.  It is independent of the HIP
library: separate C source, separate build, no shared headers or helpers.

Forms (see ``la_oracle.c`` for the page citations):

* :func:`recurrent` -- form (b), token-by-token right product with a running
  d x d fp64 state that restarts at every document start.
* :func:`quadratic` -- form (a), masked left product (tiny inputs only).
* :func:`decode_step` -- one length-1 step: state update, then read.

Each takes ``decay`` (per-head factors in [0, 1]; per pair for decode_step)
for the decayed variant S_t = lambda S_{t-1} + k_t^T v_t (a reading of the
decay the pages name but never define; ``None`` = no decay).

Inputs are numpy arrays: bf16 as uint16 bit patterns, or float32 / float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_SO = os.path.join(_HERE, "_laoracle.so")


def build(force: bool = False, out: str | None = None, extra_flags=()) -> str:
    """Compile la_oracle.c with gcc (no fast-math) into a shared library."""
    target = out or _SO
    if force or out or not os.path.exists(target) or os.path.getmtime(target) < os.path.getmtime(_SRC):
        tmp = target + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", *extra_flags, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, target)
    return target


def _bind(lib):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.ora_recurrent.argtypes = [vp, vp, vp, ctypes.c_int, vp, i32, i32, i32, i32, i32, vp, vp, vp, ctypes.c_int]
    lib.ora_quadratic.argtypes = [vp, vp, vp, ctypes.c_int, vp, i32, i32, i32, vp, vp, vp]
    lib.ora_decode_step.argtypes = [vp, vp, vp, ctypes.c_int, i64, i32, vp, vp, ctypes.c_int]
    lib.ora_backward.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_int]
    lib.ora_recurrent_decay.argtypes = [vp, vp, vp, ctypes.c_int, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                        ctypes.c_int]
    lib.ora_quadratic_decay.argtypes = [vp, vp, vp, ctypes.c_int, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.ora_decode_step_decay.argtypes = [vp, vp, vp, ctypes.c_int, i64, i32, vp, vp, vp, ctypes.c_int]
    lib.ora_last_threads.restype = ctypes.c_int
    return lib


_lib = None


def load(path: str | None = None):
    """The oracle library (built on first use).  ``path`` loads another build
    of the same source (used by the tests that plant mistakes)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = _bind(ctypes.CDLL(_SO))
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 0
    if a.dtype == np.float32:
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dt=None):
    return np.ascontiguousarray(a if dt is None else np.asarray(a, dtype=dt))


def _decay(decay, n):
    if decay is None:
        return None
    a = np.ascontiguousarray(np.asarray(decay, dtype=np.float64).reshape(-1))
    assert a.size == n, (a.size, n)
    return a


def recurrent(q, k, v, cu_seqlens, kv_in=None, want_o=True, want_state=True, heads=None,
              nthreads: int = 0, lib=None, decay=None):
    """Form (b).  q, k, v: [T, H, d].  Returns (o [T, nh, d] fp64 or None,
    kv_out [num_seqs, H, d, d] fp64 or None); with ``heads=(h0, h1)`` only that
    head range is computed (kv_out rows of other heads stay zero)."""
    lib = lib or load()
    q, k, v = _c(q), _c(k), _c(v)
    assert q.shape == k.shape == v.shape and q.ndim == 3 and q.dtype == k.dtype == v.dtype
    T, H, d = q.shape
    cu = _c(cu_seqlens, np.int32)
    D = cu.size - 1
    assert cu[-1] == T
    h0, h1 = heads if heads is not None else (0, H)
    kvi = None if kv_in is None else _c(kv_in, np.float64)
    o = np.empty((T, h1 - h0, d), dtype=np.float64) if want_o else None
    kvo = np.zeros((D, H, d, d), dtype=np.float64) if want_state else None
    lam = _decay(decay, H)
    if lam is None:
        rc = lib.ora_recurrent(_p(q), _p(k), _p(v), _dtype_code(q), _p(cu), D, H, d, h0, h1, _p(kvi), _p(o), _p(kvo),
                               nthreads)
    else:
        rc = lib.ora_recurrent_decay(_p(q), _p(k), _p(v), _dtype_code(q), _p(cu), D, H, d, h0, h1, _p(lam), _p(kvi),
                                     _p(o), _p(kvo), nthreads)
    if rc != 0:
        raise ValueError("ora_recurrent rejected its arguments")
    return o, kvo


def quadratic(q, k, v, cu_seqlens, kv_in=None, lib=None, decay=None):
    """Form (a), every head, single thread.  Returns (o, kv_out) in fp64."""
    lib = lib or load()
    q, k, v = _c(q), _c(k), _c(v)
    T, H, d = q.shape
    cu = _c(cu_seqlens, np.int32)
    D = cu.size - 1
    kvi = None if kv_in is None else _c(kv_in, np.float64)
    o = np.empty((T, H, d), dtype=np.float64)
    kvo = np.empty((D, H, d, d), dtype=np.float64)
    lam = _decay(decay, H)
    if lam is None:
        rc = lib.ora_quadratic(_p(q), _p(k), _p(v), _dtype_code(q), _p(cu), D, H, d, _p(kvi), _p(o), _p(kvo))
    else:
        rc = lib.ora_quadratic_decay(_p(q), _p(k), _p(v), _dtype_code(q), _p(cu), D, H, d, _p(lam), _p(kvi), _p(o),
                                     _p(kvo))
    if rc != 0:
        raise ValueError("ora_quadratic rejected its arguments")
    return o, kvo


def backward(q, k, v, dout, cu_seqlens, kv_in=None, dkv_out=None, want_dkv_in=True, nthreads: int = 0, lib=None):
    """Gradients of sum(dout * o) + sum(dkv_out * kv_out) for the prefill of
    (q, k, v, cu_seqlens, kv_in).  Returns fp64 (dq, dk, dv, dkv_in or None)."""
    lib = lib or load()
    q, k, v, dout = _c(q), _c(k), _c(v), _c(dout)
    assert q.shape == k.shape == v.shape == dout.shape and q.dtype == k.dtype == v.dtype == dout.dtype
    T, H, d = q.shape
    cu = _c(cu_seqlens, np.int32)
    D = cu.size - 1
    assert cu[-1] == T
    kvi = None if kv_in is None else _c(kv_in, np.float64)
    dko = None if dkv_out is None else _c(dkv_out, np.float64)
    dq, dk, dv = (np.empty((T, H, d), dtype=np.float64) for _ in range(3))
    dki = np.empty((D, H, d, d), dtype=np.float64) if want_dkv_in else None
    rc = lib.ora_backward(_p(q), _p(k), _p(v), _p(dout), _dtype_code(q), _p(cu), D, H, d, _p(kvi), _p(dko), _p(dq),
                          _p(dk), _p(dv), _p(dki), nthreads)
    if rc != 0:
        raise ValueError("ora_backward rejected its arguments")
    return dq, dk, dv, dki


def decode_step(q, k, v, S, nthreads: int = 0, lib=None, decay=None):
    """S (fp64 [P, d, d]) is updated in place; returns o fp64 [P, d].
    decay: per-pair factors [P] (the decayed variant) or None."""
    lib = lib or load()
    q, k, v = _c(q), _c(k), _c(v)
    d = q.shape[-1]
    P = q.size // d
    assert S.dtype == np.float64 and S.flags.c_contiguous and S.size == P * d * d
    o = np.empty((P, d), dtype=np.float64)
    lam = _decay(decay, P)
    if lam is None:
        rc = lib.ora_decode_step(_p(q), _p(k), _p(v), _dtype_code(q), P, d, _p(S), _p(o), nthreads)
    else:
        rc = lib.ora_decode_step_decay(_p(q), _p(k), _p(v), _dtype_code(q), P, d, _p(lam), _p(S), _p(o), nthreads)
    if rc != 0:
        raise ValueError("ora_decode_step rejected its arguments")
    return o


def last_threads(lib=None) -> int:
    return int((lib or load()).ora_last_threads())
