"""fp64 CPU oracle for the fused feed-forward network -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or runs anything here, and this
package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only
marshals numpy arrays into it.  What it computes, with its sources:

* ``ffn``: ``Y = act2(act1(X W1 + b1) W2 + b2)`` -- the kernel-fusion /
  tensor-parallelism post (brunomaga.github.io), section "Megatron-LM tensor
  parallelism", equations for H and Y.  With ``b2=None`` and ``act2=NONE`` it
  is one tensor-parallel shard's partial output (same section, the equation
  summing ``H^(g) W2^(g)`` over shards before b2 is added).
* ``moe_route`` / ``moe_ffn``: top-k routing and the gate-weighted sum of the
  selected experts' FFN outputs -- the MoE tile-signalling review
  (zhongzhuzhou.org), sections 2.1 and 2.2.

Build: ``gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm``
(``build()`` below, also called by ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU_TANH = 0, 1, 2

_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (OpenMP over rows)."""
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", src, "-o", out, "-lm"],
                   check=True)
    return out


def load(path: str | None = None):
    """Load (building on first use) the oracle library; ``path`` loads another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    vp, i64, i32, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_ffn.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, dp]
    lib.oracle_ffn.restype = ctypes.c_int
    lib.oracle_moe_route.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.oracle_moe_route.restype = ctypes.c_int
    lib.oracle_moe_ffn.argtypes = [i32, vp, vp, i64, i64, i32, vp, vp, vp, vp, i64, i64, i64,
                                   i32, i32, vp, i64, dp]
    lib.oracle_moe_ffn.restype = ctypes.c_int
    lib.oracle_swiglu.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, dp]
    lib.oracle_swiglu.restype = ctypes.c_int
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_router_logits.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, dp]
    lib.oracle_router_logits.restype = ctypes.c_int
    lib.oracle_act_grad.argtypes = [i32, ctypes.c_double]
    lib.oracle_act_grad.restype = ctypes.c_double
    lib.oracle_ffn_backward.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                        vp, i64, dp, vp, i64, dp, dp, dp, dp]
    lib.oracle_ffn_backward.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_act.argtypes = [i32, ctypes.c_double]
    lib.oracle_act.restype = ctypes.c_double
    return lib


def _as_input(a, dtype_code):
    """Return (contiguous array, pointer) holding the exact bits the GPU receives.

    bf16 inputs are passed as their uint16 bit patterns; fp32 as float32."""
    if a is None:
        return None, None
    a = np.ascontiguousarray(a)
    if dtype_code == BF16:
        if a.dtype != np.uint16:
            raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    elif a.dtype != np.float32:
        raise TypeError("fp32 inputs must be float32")
    return a, a.ctypes.data


def _dtype_of(X):
    return BF16 if np.asarray(X).dtype == np.uint16 else F32


def threads(lib=None) -> int:
    """OpenMP threads the oracle's row loops use."""
    return (lib or load()).oracle_threads()


def act(kind: int, x: float, lib=None) -> float:
    """The oracle's activation applied to one double (for the closed-form pins)."""
    return (lib or load()).oracle_act(kind, float(x))


def ffn(X, W1, b1, W2, b2, act1=ACT_GELU_TANH, act2=ACT_NONE, rows=None, lib=None):
    """fp64 ``Y[rows] = act2(act1(X W1 + b1) W2 + b2)``.

    ``X`` (M x N), ``W1`` (N x O), ``W2`` (O x P) and the biases are float32 arrays,
    or uint16 arrays of bf16 bit patterns.  ``rows`` selects output rows (all if None)."""
    lib = lib or load()
    dt = _dtype_of(X)
    M, N = X.shape
    O = W1.shape[1]
    P = W2.shape[1]
    assert W1.shape == (N, O) and W2.shape == (O, P)
    keep = [_as_input(a, dt) for a in (X, W1, b1, W2, b2)]
    ptr = [k[1] for k in keep]
    if rows is None:
        rws, rp, nr = None, None, M
    else:
        rws = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        rp, nr = rws.ctypes.data, rws.size
    Y = np.empty((nr, P), dtype=np.float64)
    rc = lib.oracle_ffn(dt, ptr[0], ptr[1], ptr[2], ptr[3], ptr[4], rp, nr, M, N, O, P,
                        act1, act2, Y.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_ffn rejected its arguments")
    return Y


def act_grad(kind: int, x: float, lib=None) -> float:
    """The oracle's act1 derivative at one double."""
    return (lib or load()).oracle_act_grad(kind, float(x))


def ffn_backward(X, W1, b1, W2, dY, act1=ACT_GELU_TANH, rows=None, cols=None, lib=None):
    """fp64 gradients of the FFN (act2 none) for the output gradient dY.

    Returns (dX[rows], dW1[:, cols], db1[cols], dW2[cols, :], db2) with rows/cols
    None meaning all; inputs as for ``ffn`` (dY in the same dtype as X)."""
    lib = lib or load()
    dt = _dtype_of(X)
    M, N = X.shape
    O = W1.shape[1]
    P = W2.shape[1]
    assert W1.shape == (N, O) and W2.shape == (O, P) and dY.shape == (M, P)
    keep = [None if a is None else _as_input(a, dt) for a in (X, W1, b1, W2, dY)]
    ptr = [None if k is None else k[1] for k in keep]
    def idx(v, n):
        if v is None:
            return None, None, n
        a = np.ascontiguousarray(np.asarray(v, dtype=np.int64))
        return a, a.ctypes.data, a.size
    rk, rp, nr = idx(rows, M)
    ck, cp, nc = idx(cols, O)
    dX = np.empty((nr, N), np.float64)
    dW1 = np.empty((N, nc), np.float64)
    db1 = np.empty(nc, np.float64)
    dW2 = np.empty((nc, P), np.float64)
    db2 = np.empty(P, np.float64)
    rc = lib.oracle_ffn_backward(dt, ptr[0], ptr[1], ptr[2], ptr[3], ptr[4], M, N, O, P, int(act1),
                                 rp, nr, dX.ctypes.data, cp, nc, dW1.ctypes.data, db1.ctypes.data,
                                 dW2.ctypes.data, db2.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_ffn_backward rejected its arguments")
    return dX, dW1, db1, dW2, db2


def silu(x: float, lib=None) -> float:
    """The oracle's silu applied to one double (for the closed-form pins)."""
    return (lib or load()).oracle_silu(float(x))


def swiglu(X, Wg, Wu, Wd, rows=None, lib=None):
    """fp64 ``Y[rows] = (silu(X Wg) * (X Wu)) Wd`` (the SwiGLU FFN: no biases).

    ``X`` (M x N), ``Wg`` and ``Wu`` (N x O), ``Wd`` (O x P): float32 arrays or uint16
    arrays of bf16 bit patterns."""
    lib = lib or load()
    dt = _dtype_of(X)
    M, N = X.shape
    O = Wg.shape[1]
    P = Wd.shape[1]
    assert Wg.shape == (N, O) and Wu.shape == (N, O) and Wd.shape == (O, P)
    keep = [_as_input(a, dt) for a in (X, Wg, Wu, Wd)]
    ptr = [k[1] for k in keep]
    if rows is None:
        rws, rp, nr = None, None, M
    else:
        rws = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        rp, nr = rws.ctypes.data, rws.size
    Y = np.empty((nr, P), dtype=np.float64)
    rc = lib.oracle_swiglu(dt, ptr[0], ptr[1], ptr[2], ptr[3], rp, nr, M, N, O, P, Y.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_swiglu rejected its arguments")
    return Y


def router_logits(X, Wr, br=None, rows=None, lib=None):
    """fp64 router logits ``X Wr + br`` (the gate network as one linear layer).

    ``X`` (M x N) and ``Wr`` (N x E): float32 arrays or uint16 bf16 bit patterns;
    ``br``: E float32 values or None."""
    lib = lib or load()
    dt = _dtype_of(X)
    M, N = X.shape
    E = Wr.shape[1]
    assert Wr.shape == (N, E)
    kx, kw = _as_input(X, dt), _as_input(Wr, dt)
    b = None if br is None else np.ascontiguousarray(br, dtype=np.float32)
    assert b is None or b.shape == (E,)
    if rows is None:
        rws, rp, nr = None, None, M
    else:
        rws = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        rp, nr = rws.ctypes.data, rws.size
    out = np.empty((nr, E), dtype=np.float64)
    rc = lib.oracle_router_logits(dt, kx[1], kw[1], None if b is None else b.ctypes.data, rp, nr,
                                  M, N, E, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_router_logits rejected its arguments")
    return out


def moe_route(logits, k=2, lib=None):
    """Top-k routing of fp32 logits (M x E): returns ids, weights, counts, offsets, sorted."""
    lib = lib or load()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    M, E = lg.shape
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float64)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    srt = np.empty(M * k, np.int32)
    rc = lib.oracle_moe_route(lg.ctypes.data, M, E, k, ids.ctypes.data, w.ctypes.data,
                              counts.ctypes.data, offsets.ctypes.data, srt.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_moe_route rejected its arguments")
    return ids, w, counts, offsets, srt


def moe_ffn(X, logits, W1, b1, W2, b2, k=2, act1=ACT_GELU_TANH, act2=ACT_NONE, rows=None,
            lib=None):
    """fp64 MoE output rows: ``sum_s w[t,s] FFN_{e_s}(X[t])``; weights stacked (E, ...)."""
    lib = lib or load()
    dt = _dtype_of(X)
    M, N = X.shape
    E, _, O = W1.shape
    P = W2.shape[2]
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    assert lg.shape == (M, E)
    keep = [_as_input(a, dt) for a in (X, W1, b1, W2, b2)]
    ptr = [kk[1] for kk in keep]
    if rows is None:
        rws, rp, nr = None, None, M
    else:
        rws = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        rp, nr = rws.ctypes.data, rws.size
    Y = np.empty((nr, P), dtype=np.float64)
    rc = lib.oracle_moe_ffn(dt, ptr[0], lg.ctypes.data, M, E, k, ptr[1], ptr[2], ptr[3],
                            ptr[4], N, O, P, act1, act2, rp, nr, Y.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_moe_ffn rejected its arguments")
    return Y
