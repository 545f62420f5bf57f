"""Causal linear attention (Lightning-style prefill and decode) for AMD MI355X.

Thin binding over the C ABI in ``include/la.h`` (``liblightning_la.so``, HIP
for gfx950).  The functions named like the C entry points take raw device
pointers and sizes and only marshal arguments; :func:`prefill` and
:func:`decode` take torch tensors (torch provides device memory and the
current stream, nothing else).  Every step of the computation runs in the HIP
kernels: there is no fallback path.  If the library has not been built the
import of this module still succeeds, but every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblightning_la.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_HIP = range(5)
LA_BF16, LA_FP32 = 0, 1

EXPORTED = ("la_prefill", "la_decode", "la_prefill_workspace_size", "la_status_string", "la_prefill_plan",
            "la_prefill_workspace_size_ex", "la_prefill_ex", "la_prefill_resume", "la_prefill_backward",
            "la_bench_stream", "la_prefill_noalloc", "la_prefill_decay", "la_decode_decay",
            "la_prefill_backward_workspace_size")


class LAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class la_prefill_opts(ctypes.Structure):
    _fields_ = [("seg_len", ctypes.c_int32), ("value_slices", ctypes.c_int32), ("force_scan", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("main_begin_event", ctypes.c_void_p),
                ("main_end_event", ctypes.c_void_p), ("slots", ctypes.c_int32),
                ("forward_states", ctypes.c_int32), ("work_list", ctypes.c_int32)]


class la_prefill_plan_info(ctypes.Structure):
    _fields_ = [("seg_len", ctypes.c_int32), ("value_slices", ctypes.c_int32), ("num_segments", ctypes.c_int32),
                ("scan", ctypes.c_int32), ("units", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("variant", ctypes.c_int32), ("slots", ctypes.c_int32), ("packed", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return LIB_PATH


def load():
    """The HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m causal_linear_attention_la_amd._build`")
    # torch first: the library then binds to the HIP runtime torch has already
    # loaded (same soname).  Loaded before torch, it would bring in the system
    # HIP runtime beside torch's bundled one, and torch's tensors and streams
    # would be handed to a second runtime (its launches then fail).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.la_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, i32, i64, ctypes.c_int, vp, sz, vp]
    lib.la_prefill.restype = ctypes.c_int
    lib.la_prefill_ex.argtypes = lib.la_prefill.argtypes + [ctypes.POINTER(la_prefill_opts)]
    lib.la_prefill_ex.restype = ctypes.c_int
    lib.la_prefill_resume.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, i32, i64, ctypes.c_int, vp, sz, vp,
                                      ctypes.POINTER(la_prefill_opts)]
    lib.la_prefill_resume.restype = ctypes.c_int
    lib.la_prefill_backward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, i64,
                                        ctypes.c_int, vp, sz, vp, ctypes.POINTER(la_prefill_opts)]
    lib.la_prefill_backward.restype = ctypes.c_int
    lib.la_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_int, vp]
    lib.la_decode.restype = ctypes.c_int
    lib.la_prefill_workspace_size.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int]
    lib.la_prefill_workspace_size.restype = sz
    lib.la_prefill_workspace_size_ex.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int,
                                                 ctypes.POINTER(la_prefill_opts)]
    lib.la_prefill_workspace_size_ex.restype = sz
    lib.la_prefill_backward_workspace_size.argtypes = lib.la_prefill_workspace_size_ex.argtypes
    lib.la_prefill_backward_workspace_size.restype = sz
    lib.la_prefill_plan.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int, ctypes.POINTER(la_prefill_opts),
                                    ctypes.POINTER(la_prefill_plan_info)]
    lib.la_prefill_plan.restype = ctypes.c_int
    lib.la_status_string.argtypes = [ctypes.c_int]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_prefill_decay.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, i32, i64, ctypes.c_int, vp, sz, vp,
                                     ctypes.POINTER(la_prefill_opts)]
    lib.la_prefill_decay.restype = ctypes.c_int
    lib.la_decode_decay.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_int, vp]
    lib.la_decode_decay.restype = ctypes.c_int
    lib.la_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, i32, i64, ctypes.c_int, vp]
    lib.la_prefill_noalloc.restype = ctypes.c_int
    lib.la_bench_stream.argtypes = [i32, vp, vp, vp, vp, sz, i32, i32, vp]
    lib.la_bench_stream.restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------- C-ABI mirrors

def status_string(status: int) -> str:
    return load().la_status_string(int(status)).decode()


def la_prefill(q, k, v, o, cu_seqlens, H, d, block, kv_state_out, num_seqs, total_tokens, dtype, workspace,
               workspace_bytes, stream) -> int:
    return load().la_prefill(q, k, v, o, cu_seqlens, H, d, block, kv_state_out, num_seqs, total_tokens, dtype,
                             workspace, workspace_bytes, stream)


def la_prefill_ex(q, k, v, o, cu_seqlens, H, d, block, kv_state_out, num_seqs, total_tokens, dtype, workspace,
                  workspace_bytes, stream, opts: la_prefill_opts | None) -> int:
    return load().la_prefill_ex(q, k, v, o, cu_seqlens, H, d, block, kv_state_out, num_seqs, total_tokens, dtype,
                                workspace, workspace_bytes, stream, ctypes.byref(opts) if opts is not None else None)


def la_prefill_resume(q, k, v, o, cu_seqlens, H, d, block, kv_state_in, kv_state_out, num_seqs, total_tokens, dtype,
                      workspace, workspace_bytes, stream, opts: la_prefill_opts | None) -> int:
    return load().la_prefill_resume(q, k, v, o, cu_seqlens, H, d, block, kv_state_in, kv_state_out, num_seqs,
                                    total_tokens, dtype, workspace, workspace_bytes, stream,
                                    ctypes.byref(opts) if opts is not None else None)


def la_prefill_backward(q, k, v, dout, cu_seqlens, H, d, block, kv_state_in, dkv_state_out, dq, dk, dv, dkv_state_in,
                        num_seqs, total_tokens, dtype, workspace, workspace_bytes, stream,
                        opts: la_prefill_opts | None) -> int:
    return load().la_prefill_backward(q, k, v, dout, cu_seqlens, H, d, block, kv_state_in, dkv_state_out, dq, dk, dv,
                                      dkv_state_in, num_seqs, total_tokens, dtype, workspace, workspace_bytes, stream,
                                      ctypes.byref(opts) if opts is not None else None)


def la_decode(q, k, v, kv_state_inout, o, num_seqs, H, d, dtype, stream) -> int:
    return load().la_decode(q, k, v, kv_state_inout, o, num_seqs, H, d, dtype, stream)


def la_prefill_decay(q, k, v, o, cu_seqlens, H, d, block, decay, kv_state_in, kv_state_out, num_seqs, total_tokens,
                     dtype, workspace, workspace_bytes, stream, opts: la_prefill_opts | None) -> int:
    return load().la_prefill_decay(q, k, v, o, cu_seqlens, H, d, block, decay, kv_state_in, kv_state_out, num_seqs,
                                   total_tokens, dtype, workspace, workspace_bytes, stream,
                                   ctypes.byref(opts) if opts is not None else None)


def la_decode_decay(q, k, v, decay, kv_state_inout, o, num_seqs, H, d, dtype, stream) -> int:
    return load().la_decode_decay(q, k, v, decay, kv_state_inout, o, num_seqs, H, d, dtype, stream)


def la_prefill_noalloc(q, k, v, o, cu_seqlens, H, d, block, kv_state_out, num_seqs, total_tokens, dtype,
                       stream) -> int:
    return load().la_prefill_noalloc(q, k, v, o, cu_seqlens, H, d, block, kv_state_out, num_seqs, total_tokens,
                                     dtype, stream)


def la_bench_stream(mode, a, b, c, dst, nbytes, workgroups, nontemporal, stream) -> int:
    return load().la_bench_stream(mode, a, b, c, dst, nbytes, workgroups, nontemporal, stream)


def la_prefill_workspace_size(total_tokens, num_seqs, H, d, block, dtype) -> int:
    return int(load().la_prefill_workspace_size(total_tokens, num_seqs, H, d, block, dtype))


def make_opts(seg_len: int = 0, value_slices: int = 0, force_scan: bool = False, begin_event=None,
              end_event=None, variant: int = 0, slots: int = 0, forward_states: bool = False,
              work_list: int = 0) -> la_prefill_opts:
    return la_prefill_opts(int(seg_len), int(value_slices), 1 if force_scan else 0, int(variant),
                           _event_ptr(begin_event), _event_ptr(end_event), int(slots), 1 if forward_states else 0,
                           int(work_list))


def la_prefill_workspace_size_ex(total_tokens, num_seqs, H, d, block, dtype, opts=None) -> int:
    return int(load().la_prefill_workspace_size_ex(total_tokens, num_seqs, H, d, block, dtype,
                                                   ctypes.byref(opts) if opts is not None else None))


def la_prefill_backward_workspace_size(total_tokens, num_seqs, H, d, block, dtype, opts=None) -> int:
    return int(load().la_prefill_backward_workspace_size(total_tokens, num_seqs, H, d, block, dtype,
                                                         ctypes.byref(opts) if opts is not None else None))


def la_prefill_plan(total_tokens, num_seqs, H, d, block, dtype, opts=None) -> dict:
    info = la_prefill_plan_info()
    st = load().la_prefill_plan(total_tokens, num_seqs, H, d, block, dtype,
                                ctypes.byref(opts) if opts is not None else None, ctypes.byref(info))
    if st != LA_OK:
        raise LAError(st, "la_prefill_plan")
    return dict(seg_len=info.seg_len, value_slices=info.value_slices, num_segments=info.num_segments,
                scan=info.scan, units=info.units, workspace_bytes=info.workspace_bytes, variant=info.variant,
                slots=info.slots, packed=info.packed)


# ------------------------------------------------------------ torch layer

def _event_ptr(ev):
    """hipEvent_t handle from a ctypes pointer, an int, or a torch.cuda.Event
    (which must have been recorded once, so that it exists)."""
    if ev is None:
        return None
    if isinstance(ev, ctypes.c_void_p):
        return ev
    return ctypes.c_void_p(int(ev.cuda_event) if hasattr(ev, "cuda_event") else int(ev))


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream_ptr(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check(cond: bool, exc, msg: str):
    if not cond:
        raise exc(msg)


def _check_tensors(ref, named, where: str):
    """Every tensor in `named` ({name: (tensor or None, dtype or None for
    ref's dtype, shape)}) has that dtype and shape, is contiguous and sits on
    ref's device, which is a GPU.  Checked in that order, before any pointer
    reaches the C ABI: a host pointer, a wrong dtype or a short buffer would
    otherwise be read or written by the kernels."""
    import torch

    for name, (t, dtype, shape) in named.items():
        if t is None:
            continue
        _check(isinstance(t, torch.Tensor), TypeError, f"{where}: {name} must be a torch.Tensor")
        want = ref.dtype if dtype is None else dtype
        _check(t.dtype == want, TypeError, f"{where}: {name} has dtype {t.dtype}, expected {want}")
        _check(tuple(t.shape) == tuple(shape), ValueError,
               f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        _check(t.is_contiguous(), ValueError, f"{where}: {name} must be contiguous")
        _check(t.device == ref.device, ValueError, f"{where}: {name} is on {t.device}, q is on {ref.device}")
    _check(ref.is_cuda, ValueError, f"{where}: tensors must be on a GPU (q is on {ref.device})")


def _check_cu(cu_seqlens, where: str):
    import torch

    _check(isinstance(cu_seqlens, torch.Tensor), TypeError, f"{where}: cu_seqlens must be a torch.Tensor")
    _check(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2, ValueError,
           f"{where}: cu_seqlens must be 1-D with num_seqs + 1 >= 2 entries")
    _check(cu_seqlens.dtype == torch.int32, TypeError, f"{where}: cu_seqlens must be int32, got {cu_seqlens.dtype}")


def _check_ws(ws, ref, where: str):
    import torch

    if ws is None:
        return
    _check(isinstance(ws, torch.Tensor), TypeError, f"{where}: workspace must be a torch.Tensor")
    _check(ws.is_contiguous(), ValueError, f"{where}: workspace must be contiguous")
    _check(ws.device == ref.device, ValueError, f"{where}: workspace is on {ws.device}, q is on {ref.device}")


def prefill(q, k, v, cu_seqlens, block: int = 64, want_state: bool = True, out=None, kv_state_out=None,
            workspace=None, seg_len: int = 0, value_slices: int = 0, force_scan: bool = False, stream=None,
            begin_event=None, end_event=None, variant: int = 0, kv_state_in=None, slots: int = 0,
            work_list: int = 0, decay=None):
    """Lightning-style causal linear attention over packed documents.

    q, k, v: [T, H, d] bf16/fp32 CUDA tensors; cu_seqlens: int32 [num_seqs + 1]
    CUDA tensor.  Returns (o, kv_state) with kv_state fp32 [num_seqs, H, d, d]
    (None when want_state is False).  kv_state_in (fp32 [num_seqs, H, d, d],
    optional) is each document's state before its first token (la_prefill_resume).
    Asynchronous on the current stream (or `stream`).  decay (fp32 [H] CUDA
    tensor, optional): each head's factor lambda in [0, 1] of the decayed
    variant (la_prefill_decay).
    """
    import torch

    _check(q.dim() == 3, ValueError, f"prefill: q must be [T, H, d], got shape {tuple(q.shape)}")
    T, H, d = q.shape
    dt = _dtype_code(q)
    _check_cu(cu_seqlens, "prefill")
    num_seqs = cu_seqlens.numel() - 1
    st_shape = (num_seqs, H, d, d)
    _check_tensors(q, {"k": (k, None, q.shape), "v": (v, None, q.shape), "out": (out, None, q.shape),
                       "kv_state_out": (kv_state_out, torch.float32, st_shape),
                       "kv_state_in": (kv_state_in, torch.float32, st_shape),
                       "cu_seqlens": (cu_seqlens, torch.int32, (num_seqs + 1,)),
                       "decay": (decay, torch.float32, (H,)), "q": (q, None, q.shape)},
                   "prefill")
    _check_ws(workspace, q, "prefill")
    o = out if out is not None else torch.empty_like(q)
    kv = kv_state_out
    if kv is None and want_state:
        kv = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device=q.device)
    opts = make_opts(seg_len, value_slices, force_scan, begin_event, end_event, variant, slots,
                     work_list=work_list)
    need = la_prefill_workspace_size_ex(T, num_seqs, H, d, block, dt, opts)
    ws = workspace
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    if decay is not None:
        st = la_prefill_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cu_seqlens), H, d, block, _ptr(decay),
                              _ptr(kv_state_in), _ptr(kv), num_seqs, T, dt, _ptr(ws) if need else None,
                              ws_bytes if need else 0, _stream_ptr(stream), opts)
    else:
        st = la_prefill_resume(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cu_seqlens), H, d, block, _ptr(kv_state_in),
                               _ptr(kv), num_seqs, T, dt, _ptr(ws) if need else None, ws_bytes if need else 0,
                               _stream_ptr(stream), opts)
    if st != LA_OK:
        raise LAError(st, "la_prefill_decay" if decay is not None else "la_prefill")
    return o, kv


def backward(q, k, v, dout, cu_seqlens, block: int = 64, kv_state_in=None, dkv_state_out=None,
             want_dkv_in: bool = True, workspace=None, seg_len: int = 0, value_slices: int = 0,
             force_scan: bool = False, stream=None, variant: int = 0, out=None, slots: int = 0,
             forward_workspace=None, work_list: int = 0):
    """Gradients of the prefill (la_prefill_backward).  dout is dL/do
    ([T, H, d], same dtype as q); dkv_state_out (fp32 [num_seqs, H, d, d] or
    None) is dL/dkv_state_out.  out = (dq, dk, dv, dkv_in) preallocated
    (dkv_in may be None), else they are allocated.  forward_workspace: the
    workspace the forward call on the same inputs and options used, untouched
    since; the backward then reuses (and overwrites) its segment states.  A
    workspace of la_prefill_backward_workspace_size bytes (what is allocated
    here when none is given) lets the dv and dk passes share a launch; one of
    the forward's size runs them one after the other.
    Returns (dq, dk, dv, dkv_state_in or None)."""
    import torch

    _check(q.dim() == 3, ValueError, f"backward: q must be [T, H, d], got shape {tuple(q.shape)}")
    T, H, d = q.shape
    dt = _dtype_code(q)
    _check_cu(cu_seqlens, "backward")
    num_seqs = cu_seqlens.numel() - 1
    st_shape = (num_seqs, H, d, d)
    named = {"k": (k, None, q.shape), "v": (v, None, q.shape), "dout": (dout, None, q.shape),
             "kv_state_in": (kv_state_in, torch.float32, st_shape),
             "dkv_state_out": (dkv_state_out, torch.float32, st_shape),
             "cu_seqlens": (cu_seqlens, torch.int32, (num_seqs + 1,)), "q": (q, None, q.shape)}
    if out is not None:
        _check(len(out) == 4, ValueError, "backward: out must be (dq, dk, dv, dkv_in)")
        named.update({"dq": (out[0], None, q.shape), "dk": (out[1], None, q.shape), "dv": (out[2], None, q.shape),
                      "dkv_in": (out[3], torch.float32, st_shape)})
    _check_tensors(q, named, "backward")
    _check_ws(workspace, q, "backward")
    _check_ws(forward_workspace, q, "backward")
    if out is not None:
        dq, dk, dv, dkv_in = out
    else:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dkv_in = torch.empty((num_seqs, H, d, d), dtype=torch.float32, device=q.device) if want_dkv_in else None
    opts = make_opts(seg_len, value_slices, force_scan, None, None, variant, slots, forward_workspace is not None,
                     work_list)
    need = la_prefill_workspace_size_ex(T, num_seqs, H, d, block, dt, opts)
    ws = forward_workspace if forward_workspace is not None else workspace
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        if forward_workspace is not None:
            raise ValueError("forward_workspace is smaller than this plan's workspace")
        ws = torch.empty(la_prefill_backward_workspace_size(T, num_seqs, H, d, block, dt, opts), dtype=torch.uint8,
                         device=q.device)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = la_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(cu_seqlens), H, d, block, _ptr(kv_state_in),
                             _ptr(dkv_state_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkv_in), num_seqs, T, dt,
                             _ptr(ws) if need else None, ws_bytes if need else 0, _stream_ptr(stream), opts)
    if st != LA_OK:
        raise LAError(st, "la_prefill_backward")
    return dq, dk, dv, dkv_in


def decode(q, k, v, kv_state, out=None, stream=None, decay=None):
    """One decode step; kv_state (fp32 [num_seqs, H, d, d]) is updated in place.
    q, k, v: [num_seqs, H, d].  decay (fp32 [H], optional): the decayed
    variant (la_decode_decay).  Returns o."""
    import torch

    _check(q.dim() == 3, ValueError, f"decode: q must be [num_seqs, H, d], got shape {tuple(q.shape)}")
    num_seqs, H, d = q.shape
    _dtype_code(q)
    _check(kv_state is not None, ValueError, "decode: kv_state is required")
    _check_tensors(q, {"k": (k, None, q.shape), "v": (v, None, q.shape), "out": (out, None, q.shape),
                       "kv_state": (kv_state, torch.float32, (num_seqs, H, d, d)),
                       "decay": (decay, torch.float32, (H,)), "q": (q, None, q.shape)},
                   "decode")
    o = out if out is not None else torch.empty_like(q)
    if decay is not None:
        st = la_decode_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(kv_state), _ptr(o), num_seqs, H, d,
                             _dtype_code(q), _stream_ptr(stream))
    else:
        st = la_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_state), _ptr(o), num_seqs, H, d, _dtype_code(q),
                       _stream_ptr(stream))
    if st != LA_OK:
        raise LAError(st, "la_decode_decay" if decay is not None else "la_decode")
    return o


def build():
    from . import _build

    return _build.build()
