"""The Python binding's argument checks, on the CPU.

The library receives raw pointers and sizes only, so the binding must refuse a
tensor whose shape, dtype, layout or device does not match the call before any
pointer reaches the library.  These tests build the arguments as ``meta``
tensors (shapes and dtypes, no storage) or CPU tensors: every call below must
raise in the binding, so none reaches the library or a GPU."""
from __future__ import annotations

import pytest
import torch

import transformer_ffn_fusion_amd as ffn

BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def meta(*shape, dtype=BF):
    return torch.empty(shape, dtype=dtype, device="meta")


M, N, O, P, E, K = 32, 64, 128, 72, 4, 2


def dense_args(dtype=BF):
    return dict(X=meta(M, N, dtype=dtype), W1=meta(N, O, dtype=dtype), b1=meta(O, dtype=dtype),
                W2=meta(O, P, dtype=dtype), b2=meta(P, dtype=dtype), Y=meta(M, P, dtype=dtype))


def call_dense(a):
    return ffn.ffn_forward(a["X"], a["W1"], a["b1"], a["W2"], a["b2"], a["Y"])


@pytest.mark.parametrize("name,bad,msg", [
    ("X", meta(M, N, 1), "dimensions"),
    ("W1", meta(N + 8, O), "shape"),
    ("b1", meta(O + 8), "shape"),
    ("W2", meta(O + 8, P), "shape"),
    ("b2", meta(P, 1), "shape"),
    ("Y", meta(M, P + 8), "shape"),
    ("Y", meta(M - 1, P), "shape"),
    ("W2", meta(O, P, dtype=F32), "dtype"),
    ("b1", meta(O, dtype=F32), "dtype"),
    ("Y", meta(M, P, dtype=F32), "dtype"),
    ("W1", meta(O, N).t(), "contiguous"),
    ("Y", meta(M, 2 * P)[:, ::2], "contiguous"),
    ("W1", None, "must not be None"),
    ("Y", None, "must not be None"),
])
def test_dense_forward_refuses(name, bad, msg):
    a = dense_args()
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=msg):
        call_dense(a)


def test_dense_forward_needs_gpu_tensors():
    with pytest.raises(ValueError, match="on the GPU"):
        call_dense(dense_args())   # well-formed, but on the meta device
    a = {k: torch.zeros(v.shape, dtype=v.dtype) for k, v in dense_args(F32).items()}
    with pytest.raises(ValueError, match="on the GPU"):
        call_dense(a)              # well-formed CPU tensors


def test_dense_forward_refuses_unknown_dtype_and_bad_workspace():
    a = dense_args()
    a["X"] = meta(M, N, dtype=torch.float16)
    with pytest.raises(TypeError):
        call_dense(a)
    a = dense_args()
    with pytest.raises(ValueError, match="uint8"):
        ffn.ffn_forward(a["X"], a["W1"], a["b1"], a["W2"], a["b2"], a["Y"],
                        ws=meta(1024, dtype=torch.int32))


@pytest.mark.parametrize("name,bad,msg", [
    ("Wu", meta(N, O + 8), "shape"),
    ("Wg", meta(N, O, dtype=F32), "dtype"),
    ("Wd", meta(P, O).t(), "contiguous"),
    ("Wu", None, "must not be None"),
    ("Y", meta(M, P + 8), "shape"),
])
def test_swiglu_refuses(name, bad, msg):
    a = dict(X=meta(M, N), Wg=meta(N, O), Wu=meta(N, O), Wd=meta(O, P), Y=meta(M, P))
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=msg):
        ffn.ffn_swiglu_forward(a["X"], a["Wg"], a["Wu"], a["Wd"], a["Y"])


@pytest.mark.parametrize("name,bad,msg", [
    ("dY", meta(M, P + 8), "shape"),
    ("dX", meta(M, N, dtype=F32), "dtype"),
    ("dW1", meta(N, O), "dtype"),          # weight gradients are fp32
    ("db1", meta(O + 8, dtype=F32), "shape"),
    ("dW2", meta(P, O, dtype=F32).t(), "contiguous"),
    ("db2", meta(P, dtype=BF), "dtype"),
])
def test_backward_refuses(name, bad, msg):
    a = dict(X=meta(M, N), W1=meta(N, O), b1=meta(O), W2=meta(O, P), dY=meta(M, P),
             dX=meta(M, N), dW1=meta(N, O, dtype=F32), db1=meta(O, dtype=F32),
             dW2=meta(O, P, dtype=F32), db2=meta(P, dtype=F32))
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=msg):
        ffn.ffn_backward(**a)


def moe_args():
    return dict(X=meta(M, N), logits=meta(M, E, dtype=F32), W1=meta(E, N, O), b1=meta(E, O),
                W2=meta(E, O, P), b2=meta(E, P), Y=meta(M, P), topk_ids=meta(M, K, dtype=I32),
                topk_w=meta(M, K, dtype=F32), expert_offsets=meta(E + 1, dtype=I32),
                sorted_entries=meta(M * K, dtype=I32))


@pytest.mark.parametrize("name,bad,msg", [
    ("X", meta(M, N, dtype=F32), "bfloat16"),
    ("logits", meta(M, E + 1, dtype=F32), "shape"),
    ("logits", meta(M, E), "dtype"),
    ("W1", meta(N, O), "dimensions"),
    ("W1", meta(E, N + 8, O), "shape"),
    ("b1", meta(E, O + 8), "shape"),
    ("W2", meta(E, O + 8, P), "shape"),
    ("b2", meta(E + 1, P), "shape"),
    ("Y", meta(M, P, dtype=F32), "dtype"),
    ("topk_ids", meta(M, K, dtype=torch.int64), "dtype"),
    ("topk_w", meta(M, K + 1, dtype=F32), "shape"),
    ("expert_offsets", meta(E, dtype=I32), "shape"),
    ("sorted_entries", meta(M, K, dtype=I32), "shape"),
    ("W2", meta(E, P, O).transpose(1, 2), "contiguous"),
])
def test_moe_forward_refuses(name, bad, msg):
    a = moe_args()
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=msg):
        ffn.moe_ffn_forward(a["X"], a["logits"], K, a["W1"], a["b1"], a["W2"], a["b2"], a["Y"],
                            topk_ids=a["topk_ids"], topk_w=a["topk_w"],
                            expert_offsets=a["expert_offsets"], sorted_entries=a["sorted_entries"])


def test_moe_forward_needs_gpu_tensors():
    a = moe_args()
    with pytest.raises(ValueError, match="on the GPU"):
        ffn.moe_ffn_forward(a["X"], a["logits"], K, a["W1"], a["b1"], a["W2"], a["b2"], a["Y"])


@pytest.mark.parametrize("name,bad,msg", [
    ("Wr", meta(N + 8, E), "shape"),
    ("Wr", meta(N, E, dtype=F32), "dtype"),
    ("br", meta(E), "dtype"),
    ("logits_out", meta(M, E + 1, dtype=F32), "shape"),
])
def test_router_refuses(name, bad, msg):
    a = dict(X=meta(M, N), Wr=meta(N, E), br=meta(E, dtype=F32), logits_out=meta(M, E, dtype=F32))
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=msg):
        ffn.moe_router(a["X"], a["Wr"], a["br"], K, logits_out=a["logits_out"])
    m = moe_args()
    with pytest.raises((ValueError, TypeError), match=msg):
        ffn.moe_ffn_forward_router(m["X"], a["Wr"], a["br"], K, m["W1"], m["b1"], m["W2"], m["b2"],
                                   m["Y"], logits_out=a["logits_out"])


@pytest.mark.parametrize("bad,msg", [
    (meta(M, E + 1, dtype=F32), None),
    (meta(M, E), "dtype"),
    (meta(E, M, dtype=F32).t(), "contiguous"),
])
def test_route_refuses(bad, msg):
    offs = meta(E + 1, dtype=I32)
    if msg is None:   # logits fine in themselves, but the offsets do not match their width
        with pytest.raises(ValueError, match="shape"):
            ffn.moe_route(bad, K, expert_offsets=offs)
    else:
        with pytest.raises((ValueError, TypeError), match=msg):
            ffn.moe_route(bad, K)
