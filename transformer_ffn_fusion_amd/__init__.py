"""Fused two-layer FFN (and its grouped MoE form) on AMD Instinct MI355X.

Thin Python binding over ``libffn.so`` (C ABI in ``include/ffn.h``).  The
functions here only marshal torch tensors into pointers, sizes and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no CPU or PyTorch fallback: if the library is missing, or a
call fails, an exception is raised.

Names mirror the C entry points: ``ffn_forward``, ``ffn_forward_ex``,
``ffn_workspace_size``, ``moe_route``, ``moe_ffn_forward``,
``moe_workspace_size``, ``ffn_last_error``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "F32", "BF16", "ACT_NONE", "ACT_RELU", "ACT_GELU_TANH",
    "VARIANT_AUTO", "VARIANT_FUSED", "VARIANT_SKINNY", "VARIANT_F32", "VARIANT_DECODE",
    "FFNError", "lib", "lib_path", "ffn_workspace_size", "ffn_forward", "ffn_forward_ex",
    "ffn_forward_family",
    "ffn_forward_noalloc", "NOALLOC_SCRATCH_BYTES",
    "moe_workspace_size", "moe_route", "moe_ffn_forward", "ffn_last_error", "workspace",
]

F32, BF16 = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU_TANH = 0, 1, 2
VARIANT_AUTO, VARIANT_FUSED, VARIANT_SKINNY, VARIANT_F32, VARIANT_DECODE = 0, 1, 2, 3, 4
ACTS = {"none": ACT_NONE, "relu": ACT_RELU, "gelu_tanh": ACT_GELU_TANH}
NOALLOC_SCRATCH_BYTES = 16 << 20   # FFN_NOALLOC_SCRATCH_BYTES in include/ffn.h

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libffn.so")
_lib = None


class FFNError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libffn error {code}: {msg}")
        self.code = code


def lib():
    """The loaded libffn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise FFNError(-100, f"{lib_path} is missing; run `python -m transformer_ffn_fusion_amd.build`")
        L = ctypes.CDLL(lib_path)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.ffn_workspace_size.argtypes = [i64, i64, i64, i64, i32]
        L.ffn_workspace_size.restype = sz
        L.ffn_workspace_size_ex.argtypes = [i64, i64, i64, i64, i32, i32]
        L.ffn_workspace_size_ex.restype = sz
        L.ffn_forward_family.argtypes = [i64, i64, i64, i64, i32, i32]
        L.ffn_forward_family.restype = i32
        L.ffn_forward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp, sz, vp]
        L.ffn_forward.restype = i32
        L.ffn_forward_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, i32,
                                     vp, sz, vp]
        L.ffn_forward_ex.restype = i32
        L.ffn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32,
                                          i32, i32, vp]
        L.ffn_forward_noalloc.restype = i32
        L.moe_workspace_size.argtypes = [i64, i64, i32, i64, i64, i64, i32]
        L.moe_workspace_size.restype = sz
        L.moe_route.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_route.restype = i32
        L.moe_ffn_forward.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp, vp, vp, i64, i64, i64, i32,
                                      i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_ffn_forward.restype = i32
        evp = ctypes.POINTER(ctypes.c_void_p)
        L.ffn_forward_traced.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32,
                                         i32, vp, sz, vp, evp, i32]
        L.ffn_forward_traced.restype = i32
        L.moe_ffn_forward_traced.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp, vp, vp, i64, i64,
                                             i64, i32, i32, i32, vp, sz, vp, evp, i32]
        L.moe_ffn_forward_traced.restype = i32
        L.ffn_swiglu_workspace_size.argtypes = [i64, i64, i64, i64, i32, i32]
        L.ffn_swiglu_workspace_size.restype = sz
        L.ffn_swiglu_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp, sz, vp]
        L.ffn_swiglu_forward.restype = i32
        L.ffn_swiglu_forward_traced.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp,
                                                sz, vp, ctypes.POINTER(vp), i32]
        L.ffn_swiglu_forward_traced.restype = i32
        L.moe_router.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_router.restype = i32
        L.moe_ffn_forward_router.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, vp, vp, vp, i64, i64,
                                             i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_ffn_forward_router.restype = i32
        L.ffn_backward_workspace_size.argtypes = [i64, i64, i64, i64, i32]
        L.ffn_backward_workspace_size.restype = sz
        L.ffn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                   i32, vp, sz, vp]
        L.ffn_backward.restype = i32
        L.ffn_backward_traced.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                          i32, i32, vp, sz, vp, ctypes.POINTER(vp), i32]
        L.ffn_backward_traced.restype = i32
        L.ffn_last_error.argtypes = []
        L.ffn_last_error.restype = ctypes.c_char_p
        L.ffn_version.restype = i32
        L.ffn_selftest_layout.restype = i32
        L.ffn_selftest_decode_expiry.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                                 i32, vp, sz, vp]
        L.ffn_selftest_decode_expiry.restype = i32
        L.ffn_ceiling_sink_bytes.argtypes = []
        L.ffn_ceiling_sink_bytes.restype = sz
        L.ffn_ceiling_mfma.argtypes = [vp, sz, i32, ctypes.POINTER(ctypes.c_double), vp]
        L.ffn_ceiling_mfma.restype = i32
        L.ffn_ceiling_read.argtypes = [vp, sz, vp, sz, vp]
        L.ffn_ceiling_read.restype = i32
        _lib = L
    return _lib


def ffn_last_error() -> str:
    return lib().ffn_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise FFNError(rc, ffn_last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _act(a):
    return ACTS[a] if isinstance(a, str) else int(a)


# ---------------------------------------------------------------- argument checks
#
# The library receives raw pointers and sizes only, so a tensor of the wrong
# shape, dtype or layout would make its kernels read or write out of bounds.
# Every wrapper checks its tensors here before anything reaches the library.

def _dims(t, name, ndim):
    if t is None:
        raise ValueError(f"{name} must not be None")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got shape {tuple(t.shape)})")
    return tuple(t.shape)


def _arg(t, name, shape, dtype, optional=False):
    """One tensor argument: shape, dtype and row-major contiguity."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} must not be None")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def _ws_arg(ws):
    import torch
    if ws is None:
        return
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous 1-D uint8 tensor")


def _on_device(*ts):
    """Every given tensor on the current GPU (the library launches there)."""
    import torch
    dev = None
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"every tensor must be on the GPU (got one on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")
    if dev is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"tensors are on {dev}, the current device is cuda:{torch.cuda.current_device()}")


def _torch_dtype(code):
    import torch
    return torch.bfloat16 if code == BF16 else torch.float32


def ffn_workspace_size(M, N, O, P, dtype=BF16, variant=VARIANT_AUTO) -> int:
    return lib().ffn_workspace_size_ex(M, N, O, P, dtype, variant)


def moe_workspace_size(M, E, k, N, O, P, dtype=BF16) -> int:
    return lib().moe_workspace_size(M, E, k, N, O, P, dtype)


def ffn_forward_family(M, N, O, P, dtype=BF16, variant=VARIANT_AUTO) -> int:
    """The kernel family (VARIANT_FUSED, _SKINNY, _F32 or _DECODE) that ``ffn_forward_ex``
    runs for this shape on the current device."""
    rc = lib().ffn_forward_family(M, N, O, P, dtype, variant)
    if rc < 0:
        raise FFNError(rc, ffn_last_error())
    return rc


def workspace(nbytes: int, device="cuda"):
    """A zero-filled device workspace of ``nbytes`` (torch allocations are 256-byte aligned)."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _dense_args(X, W1, b1, W2, b2, Y, ws=None):
    """Checks the dense call's tensors; returns M, N, O, P and the dtype code."""
    M, N = _dims(X, "X", 2)
    O = _dims(W1, "W1", 2)[1]
    P = _dims(W2, "W2", 2)[1]
    dt = _dtype_code(X)
    tdt = _torch_dtype(dt)
    _arg(X, "X", (M, N), tdt)
    _arg(W1, "W1", (N, O), tdt)
    _arg(b1, "b1", (O,), tdt, optional=True)
    _arg(W2, "W2", (O, P), tdt)
    _arg(b2, "b2", (P,), tdt, optional=True)
    _arg(Y, "Y", (M, P), tdt)
    _ws_arg(ws)
    _on_device(X, W1, b1, W2, b2, Y, ws)
    return M, N, O, P, dt


def ffn_forward_noalloc(X, W1, b1, W2, b2, Y, act1="gelu_tanh", act2="none",
                        variant=VARIANT_AUTO, stream=None):
    """As ``ffn_forward_ex`` with the library's static device scratch as the workspace:
    nothing is allocated (the shape's workspace must fit FFN_NOALLOC_SCRATCH_BYTES)."""
    M, N, O, P, dt = _dense_args(X, W1, b1, W2, b2, Y)
    _check(lib().ffn_forward_noalloc(_ptr(X), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(Y),
                                     M, N, O, P, dt, _act(act1), _act(act2), int(variant),
                                     _stream(stream)))
    return Y


def ffn_forward_ex(X, W1, b1, W2, b2, Y, act1="gelu_tanh", act2="none", variant=VARIANT_AUTO,
                   ws=None, stream=None):
    """``Y = act2(act1(X W1 + b1) W2 + b2)`` on the GPU; ``Y`` is written in place.

    ``ws`` is a zero-initialised uint8 device tensor of at least
    ``ffn_workspace_size(...)`` bytes (allocated here when None)."""
    M, N, O, P, dt = _dense_args(X, W1, b1, W2, b2, Y, ws)
    if ws is None:
        ws = workspace(ffn_workspace_size(M, N, O, P, dt, variant), X.device)
    _check(lib().ffn_forward_ex(_ptr(X), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(Y),
                                M, N, O, P, dt, _act(act1), _act(act2), int(variant),
                                _ptr(ws), ws.numel(), _stream(stream)))
    return Y


def ffn_forward(X, W1, b1, W2, b2, Y, act1="gelu_tanh", act2="none", ws=None, stream=None):
    return ffn_forward_ex(X, W1, b1, W2, b2, Y, act1, act2, VARIANT_AUTO, ws, stream)


def ffn_backward_workspace_size(M, N, O, P, dtype=BF16) -> int:
    return lib().ffn_backward_workspace_size(M, N, O, P, dtype)


def ffn_backward(X, W1, b1, W2, dY, dX, dW1, db1, dW2, db2, act1="gelu_tanh", ws=None, stream=None):
    """Gradients of the FFN (act2 none) for the output gradient ``dY``; writes dX (bf16),
    dW1, db1, dW2, db2 (fp32; db1/db2 may be None) in place."""
    import torch
    M, N = _dims(X, "X", 2)
    O = _dims(W1, "W1", 2)[1]
    P = _dims(W2, "W2", 2)[1]
    dt = _dtype_code(X)
    bf, f32 = torch.bfloat16, torch.float32
    _arg(X, "X", (M, N), bf)
    _arg(W1, "W1", (N, O), bf)
    _arg(b1, "b1", (O,), bf, optional=True)
    _arg(W2, "W2", (O, P), bf)
    _arg(dY, "dY", (M, P), bf)
    _arg(dX, "dX", (M, N), bf)
    _arg(dW1, "dW1", (N, O), f32)
    _arg(db1, "db1", (O,), f32, optional=True)
    _arg(dW2, "dW2", (O, P), f32)
    _arg(db2, "db2", (P,), f32, optional=True)
    _ws_arg(ws)
    _on_device(X, W1, b1, W2, dY, dX, dW1, db1, dW2, db2, ws)
    if ws is None:
        ws = workspace(ffn_backward_workspace_size(M, N, O, P, dt), X.device)
    _check(lib().ffn_backward(_ptr(X), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(dY), _ptr(dX), _ptr(dW1),
                              _ptr(db1), _ptr(dW2), _ptr(db2), M, N, O, P, dt, _act(act1),
                              _ptr(ws), ws.numel(), _stream(stream)))


def ffn_swiglu_workspace_size(M, N, O, P, dtype=BF16, variant=VARIANT_AUTO) -> int:
    return lib().ffn_swiglu_workspace_size(M, N, O, P, dtype, variant)


def ffn_swiglu_forward(X, Wg, Wu, Wd, Y, variant=VARIANT_AUTO, ws=None, stream=None):
    """``Y = (silu(X Wg) * (X Wu)) Wd`` on the GPU; ``Y`` is written in place."""
    M, N = _dims(X, "X", 2)
    O = _dims(Wg, "Wg", 2)[1]
    P = _dims(Wd, "Wd", 2)[1]
    dt = _dtype_code(X)
    tdt = _torch_dtype(dt)
    _arg(X, "X", (M, N), tdt)
    _arg(Wg, "Wg", (N, O), tdt)
    _arg(Wu, "Wu", (N, O), tdt)
    _arg(Wd, "Wd", (O, P), tdt)
    _arg(Y, "Y", (M, P), tdt)
    _ws_arg(ws)
    _on_device(X, Wg, Wu, Wd, Y, ws)
    if ws is None:
        ws = workspace(ffn_swiglu_workspace_size(M, N, O, P, dt, variant), X.device)
    _check(lib().ffn_swiglu_forward(_ptr(X), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(Y), M, N, O, P,
                                    dt, int(variant), _ptr(ws), ws.numel(), _stream(stream)))
    return Y


def _route_outputs(M, E, k, topk_ids, topk_w, expert_offsets, sorted_entries):
    import torch
    _arg(topk_ids, "topk_ids", (M, k), torch.int32, optional=True)
    _arg(topk_w, "topk_w", (M, k), torch.float32, optional=True)
    _arg(expert_offsets, "expert_offsets", (E + 1,), torch.int32, optional=True)
    _arg(sorted_entries, "sorted_entries", (M * k,), torch.int32, optional=True)


def _experts(X, W1, b1, W2, b2, Y):
    """Shapes of the grouped form's tensors: returns M, N, E, O, P."""
    M, N = _dims(X, "X", 2)
    E, _, O = _dims(W1, "W1", 3)
    P = _dims(W2, "W2", 3)[2]
    bf = _torch_dtype(BF16)
    if X.dtype != bf:
        raise TypeError(f"X has dtype {X.dtype}; the grouped form takes bfloat16")
    _arg(X, "X", (M, N), bf)
    _arg(W1, "W1", (E, N, O), bf)
    _arg(b1, "b1", (E, O), bf, optional=True)
    _arg(W2, "W2", (E, O, P), bf)
    _arg(b2, "b2", (E, P), bf, optional=True)
    _arg(Y, "Y", (M, P), bf)
    return M, N, E, O, P


def moe_route(logits, k, topk_ids=None, topk_w=None, expert_offsets=None, sorted_entries=None,
              ws=None, stream=None):
    """Top-k routing on the GPU; fills whichever output tensors are given."""
    import torch
    M, E = _dims(logits, "logits", 2)
    _arg(logits, "logits", (M, E), torch.float32)
    _route_outputs(M, E, k, topk_ids, topk_w, expert_offsets, sorted_entries)
    _ws_arg(ws)
    _on_device(logits, topk_ids, topk_w, expert_offsets, sorted_entries, ws)
    if ws is None:
        ws = workspace(moe_workspace_size(M, E, k, 8, 8, 8), logits.device)
    _check(lib().moe_route(_ptr(logits), M, E, k, _ptr(topk_ids), _ptr(topk_w),
                           _ptr(expert_offsets), _ptr(sorted_entries), _ptr(ws), ws.numel(),
                           _stream(stream)))


def moe_ffn_forward(X, logits, k, W1, b1, W2, b2, Y, act1="gelu_tanh", act2="none",
                    topk_ids=None, topk_w=None, expert_offsets=None, sorted_entries=None,
                    ws=None, stream=None):
    """Grouped FFN over the top-k experts of each token; ``Y`` written in place."""
    import torch
    M, N, E, O, P = _experts(X, W1, b1, W2, b2, Y)
    _arg(logits, "logits", (M, E), torch.float32)
    _route_outputs(M, E, k, topk_ids, topk_w, expert_offsets, sorted_entries)
    _ws_arg(ws)
    _on_device(X, logits, W1, b1, W2, b2, Y, topk_ids, topk_w, expert_offsets, sorted_entries, ws)
    dt = BF16
    if ws is None:
        ws = workspace(moe_workspace_size(M, E, k, N, O, P, dt), X.device)
    _check(lib().moe_ffn_forward(_ptr(X), _ptr(logits), M, E, k, _ptr(W1), _ptr(b1), _ptr(W2),
                                 _ptr(b2), _ptr(Y), N, O, P, dt, _act(act1), _act(act2),
                                 _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets),
                                 _ptr(sorted_entries), _ptr(ws), ws.numel(), _stream(stream)))
    return Y


def moe_router(X, Wr, br, k, logits_out=None, topk_ids=None, topk_w=None, expert_offsets=None,
               sorted_entries=None, ws=None, stream=None):
    """Router logits X Wr + br and top-k routing on the GPU; fills the given outputs."""
    import torch
    M, N = _dims(X, "X", 2)
    E = _dims(Wr, "Wr", 2)[1]
    _arg(X, "X", (M, N), torch.bfloat16)
    _arg(Wr, "Wr", (N, E), torch.bfloat16)
    _arg(br, "br", (E,), torch.float32, optional=True)
    _arg(logits_out, "logits_out", (M, E), torch.float32, optional=True)
    _route_outputs(M, E, k, topk_ids, topk_w, expert_offsets, sorted_entries)
    _ws_arg(ws)
    _on_device(X, Wr, br, logits_out, topk_ids, topk_w, expert_offsets, sorted_entries, ws)
    if ws is None:
        ws = workspace(moe_workspace_size(M, E, k, N, 8, 8), X.device)
    _check(lib().moe_router(_ptr(X), _ptr(Wr), _ptr(br), M, N, E, k, _ptr(logits_out),
                            _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets),
                            _ptr(sorted_entries), _ptr(ws), ws.numel(), _stream(stream)))


def moe_ffn_forward_router(X, Wr, br, k, W1, b1, W2, b2, Y, act1="gelu_tanh", act2="none",
                           logits_out=None, topk_ids=None, topk_w=None, expert_offsets=None,
                           sorted_entries=None, ws=None, stream=None):
    """The MoE layer with the router on the GPU; ``Y`` written in place."""
    import torch
    M, N, E, O, P = _experts(X, W1, b1, W2, b2, Y)
    _arg(Wr, "Wr", (N, E), torch.bfloat16)
    _arg(br, "br", (E,), torch.float32, optional=True)
    _arg(logits_out, "logits_out", (M, E), torch.float32, optional=True)
    _route_outputs(M, E, k, topk_ids, topk_w, expert_offsets, sorted_entries)
    _ws_arg(ws)
    _on_device(X, Wr, br, W1, b1, W2, b2, Y, logits_out, topk_ids, topk_w, expert_offsets,
               sorted_entries, ws)
    dt = BF16
    if ws is None:
        ws = workspace(moe_workspace_size(M, E, k, N, O, P, dt), X.device)
    _check(lib().moe_ffn_forward_router(_ptr(X), _ptr(Wr), _ptr(br), M, E, k, _ptr(W1), _ptr(b1),
                                        _ptr(W2), _ptr(b2), _ptr(Y), N, O, P, dt, _act(act1),
                                        _act(act2), _ptr(logits_out), _ptr(topk_ids), _ptr(topk_w),
                                        _ptr(expert_offsets), _ptr(sorted_entries), _ptr(ws),
                                        ws.numel(), _stream(stream)))
    return Y


# ---------------------------------------------------------------- measurement support

def ceiling_mfma(sink, iters, stream=None) -> float:
    """Enqueue the bf16 MFMA loop kernel; returns the FLOP count of the launch."""
    _on_device(sink)
    f = ctypes.c_double()
    _check(lib().ffn_ceiling_mfma(_ptr(sink), sink.numel() * sink.element_size(), iters,
                                  ctypes.byref(f), _stream(stream)))
    return f.value


def ceiling_read(src, sink, stream=None) -> int:
    """Enqueue one streaming read of ``src`` (a device tensor); returns the bytes read."""
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    _on_device(src, sink)
    nbytes = src.numel() * src.element_size()
    _check(lib().ffn_ceiling_read(_ptr(src), nbytes, _ptr(sink), sink.numel() * sink.element_size(),
                                  _stream(stream)))
    return nbytes
