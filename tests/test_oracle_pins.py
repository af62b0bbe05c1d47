"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin ties one part of the oracle to what the pages or mathematics fix:
exact rational brute force, closed forms, identities and invariants stated on
the pages, and printed sizes.  A planted mistake in any part of the oracle
(dropped bias, wrong sign, transposed index, wrong constant, wrong tie rule)
must fail at least one of them: ``test_mutants_are_caught`` builds mutated
copies of the oracle on the CPU and checks exactly that.
"""
from __future__ import annotations

import json
import math
import os
import shutil
from fractions import Fraction

import numpy as np
import pytest

import oracle
from transformer_ffn_fusion_amd import synth, workload

HERE = os.path.dirname(os.path.abspath(__file__))
NONE, RELU, GELU = oracle.ACT_NONE, oracle.ACT_RELU, oracle.ACT_GELU_TANH


# ----------------------------------------------------------------------------
# helpers (pure Python, independent of the oracle)
# ----------------------------------------------------------------------------

def _dyadic(rng, shape):
    """Values k/8 with |k| <= 16: exact in bf16, fp32 and fp64, and every
    product and short sum of them is exact in fp64."""
    return (rng.integers(-16, 17, size=shape) / 8.0).astype(np.float32)


def _frac_ffn(X, W1, b1, W2, b2, relu):
    """Exact rational FFN with Python Fractions (definition written out)."""
    M, N = X.shape
    O = W1.shape[1]
    P = W2.shape[1]
    F = lambda v: Fraction(float(v))  # noqa: E731 -- exact for these inputs
    Y = []
    for m in range(M):
        h = []
        for o in range(O):
            a = sum((F(X[m, n]) * F(W1[n, o]) for n in range(N)), Fraction(0))
            a += F(b1[o]) if b1 is not None else 0
            h.append(max(a, Fraction(0)) if relu else a)
        row = []
        for p in range(P):
            a = sum((h[o] * F(W2[o, p]) for o in range(O)), Fraction(0))
            a += F(b2[p]) if b2 is not None else 0
            row.append(a)
        Y.append(row)
    return Y


def _to_bf16(a):
    return synth.f32_to_bf16_bits(a)


# ----------------------------------------------------------------------------
# 1. exact brute force on tiny shapes
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2, 3, 4, 2), (3, 5, 7, 4), (1, 1, 1, 1), (4, 8, 3, 5)])
@pytest.mark.parametrize("relu", [True, False])
@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("as_bf16", [False, True])
def test_brute_force_exact(shape, relu, bias, as_bf16):
    M, N, O, P = shape
    rng = np.random.default_rng(hash((shape, relu, bias)) % 2**32)
    X, W1, b1, W2, b2 = (_dyadic(rng, s) for s in [(M, N), (N, O), (O,), (O, P), (P,)])
    if not bias:
        b1 = b2 = None
    exact = _frac_ffn(X, W1, b1, W2, b2, relu)
    conv = _to_bf16 if as_bf16 else (lambda a: a)
    args = [None if a is None else conv(a) for a in (X, W1, b1, W2, b2)]
    Y = oracle.ffn(*args, act1=RELU if relu else NONE, act2=NONE)
    for m in range(M):
        for p in range(P):
            assert Y[m, p] == float(exact[m][p]), (m, p, Y[m, p], exact[m][p])


def test_second_activation_relu_exact():
    """act2 applies after b2 (tensor-parallel equation: bias then activation)."""
    rng = np.random.default_rng(7)
    X, W1, b1, W2, b2 = (_dyadic(rng, s) for s in [(3, 4), (4, 5), (5,), (5, 6), (6,)])
    exact = _frac_ffn(X, W1, b1, W2, b2, relu=True)
    Y = oracle.ffn(X, W1, b1, W2, b2, act1=RELU, act2=RELU)
    for m in range(3):
        for p in range(6):
            assert Y[m, p] == float(max(exact[m][p], Fraction(0)))


# ----------------------------------------------------------------------------
# 2. closed forms with identity weights
# ----------------------------------------------------------------------------

def test_relu_identity_closed_form():
    """N=O=P, W1=W2=I, b1=0: Y = max(X, 0) + b2 exactly; negatives vanish."""
    n = 16
    rng = np.random.default_rng(3)
    X = rng.standard_normal((9, n)).astype(np.float32)
    b2 = rng.standard_normal(n).astype(np.float32)
    eye = np.eye(n, dtype=np.float32)
    Y = oracle.ffn(X, eye, np.zeros(n, np.float32), eye, b2, act1=RELU)
    expect = np.maximum(X.astype(np.float64), 0.0) + b2.astype(np.float64)
    assert np.array_equal(Y, expect)
    Yn = oracle.ffn(X, eye, None, eye, None, act1=RELU)
    assert np.all(Yn[X < 0] == 0.0)


def _gelu_sigmoid_form(x):
    # 0.5 (1 + tanh u) = 1 / (1 + exp(-2u)), u = sqrt(2/pi) (x + 0.044715 x^3)
    u = math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)
    if -2 * u > 700:
        return 0.0
    return x / (1.0 + math.exp(-2.0 * u))


def _gelu_erf(x):
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def test_gelu_tanh_pins():
    assert oracle.act(GELU, 0.0) == 0.0
    xs = np.linspace(-8, 8, 321)
    for x in xs:
        g = oracle.act(GELU, x)
        # odd-part identity: gelu(x) - gelu(-x) = x
        assert abs((g - oracle.act(GELU, -x)) - x) <= 4 * np.spacing(max(abs(x), 1.0))
        # same function through the sigmoid route (exp instead of tanh)
        assert abs(g - _gelu_sigmoid_form(x)) <= 1e-14 * max(1.0, abs(x))
        # the tanh form approximates the exact (erf) GELU closely everywhere
        assert abs(g - _gelu_erf(x)) < 1e-3
    for x in (10.0, 20.0, 50.0):
        assert abs(oracle.act(GELU, x) - x) <= 1e-15 * x
        assert abs(oracle.act(GELU, -x)) <= 1e-15
    # the identity-weight case: Y = gelu(X) + b2
    n = 8
    rng = np.random.default_rng(4)
    X = rng.standard_normal((5, n)).astype(np.float32)
    b2 = rng.standard_normal(n).astype(np.float32)
    eye = np.eye(n, dtype=np.float32)
    Y = oracle.ffn(X, eye, None, eye, b2, act1=GELU)
    expect = np.vectorize(_gelu_sigmoid_form)(X.astype(np.float64)) + b2.astype(np.float64)
    np.testing.assert_allclose(Y, expect, rtol=1e-13, atol=1e-14)


def test_relu_pins():
    assert oracle.act(RELU, -1.5) == 0.0
    assert oracle.act(RELU, 2.25) == 2.25
    assert oracle.act(RELU, 0.0) == 0.0
    assert oracle.act(NONE, -3.5) == -3.5


# ----------------------------------------------------------------------------
# 3. the no-activation collapse (Step 1 equation)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_linear_collapse(dtype):
    """act=NONE: (X W1 + b1) W2 + b2 == X (W1 W2) + (b1 W2 + b2), other association."""
    M, N, O, P = 7, 24, 40, 16
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype=dtype, bias_var=0.5, seed=11)
    Y = oracle.ffn(X, W1, b1, W2, b2, act1=NONE)
    wid = synth.bf16_bits_to_f32 if dtype == "bf16" else (lambda a: a)
    x, w1, c1, w2, c2 = (wid(a).astype(np.float64) for a in (X, W1, b1, W2, b2))
    other = x @ (w1 @ w2) + (c1 @ w2 + c2)
    np.testing.assert_allclose(Y, other, rtol=1e-12, atol=1e-12 * np.abs(other).max())


# ----------------------------------------------------------------------------
# 4. tensor-parallel invariant (sum over shards, b2 once)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("act", [RELU, GELU])
def test_tensor_parallel_invariant(G, act):
    M, N, O, P = 6, 32, 64, 24
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype="bf16", seed=5)
    full = oracle.ffn(X, W1, b1, W2, b2, act1=act)
    w = O // G
    total = np.zeros_like(full)
    for g in range(G):
        sl = slice(g * w, (g + 1) * w)
        total += oracle.ffn(X, np.ascontiguousarray(W1[:, sl]), b1[sl],
                            np.ascontiguousarray(W2[sl, :]), None, act1=act)
    total += synth.bf16_bits_to_f32(b2).astype(np.float64)
    np.testing.assert_allclose(total, full, rtol=1e-12, atol=1e-12 * np.abs(full).max())


# ----------------------------------------------------------------------------
# 5. row independence
# ----------------------------------------------------------------------------

def test_row_permutation_and_subset_bit_exact():
    M, N, O, P = 12, 16, 24, 8
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype="bf16", seed=9)
    Y = oracle.ffn(X, W1, b1, W2, b2, act1=GELU)
    perm = np.random.default_rng(2).permutation(M)
    Yp = oracle.ffn(np.ascontiguousarray(X[perm]), W1, b1, W2, b2, act1=GELU)
    assert np.array_equal(Yp, Y[perm])
    rows = [11, 0, 5]
    assert np.array_equal(oracle.ffn(X, W1, b1, W2, b2, act1=GELU, rows=rows), Y[rows])


# ----------------------------------------------------------------------------
# 6. MoE routing and combine
# ----------------------------------------------------------------------------

def _independent_topk(logits, k):
    # stable sort on -logit: among equal logits the smaller expert index comes first
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


@pytest.mark.parametrize("E,k", [(8, 2), (4, 1), (5, 3), (8, 8)])
def test_routing_matches_independent_sort(E, k):
    rng = np.random.default_rng(E * 10 + k)
    M = 257
    # coarse values force many exact ties
    logits = (rng.integers(-3, 4, size=(M, E)) * 0.5).astype(np.float32)
    ids, w, counts, offsets, srt = oracle.moe_route(logits, k=k)
    assert np.array_equal(ids, _independent_topk(logits, k))
    # weights: softmax over the selected logits, written independently
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1)
    ref = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref /= ref.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-14, atol=0)
    # grouping invariants
    assert counts.sum() == M * k and offsets[-1] == M * k and offsets[0] == 0
    assert np.array_equal(np.diff(offsets), counts)
    flat = ids.reshape(-1)
    assert np.array_equal(srt, np.argsort(flat, kind="stable").astype(np.int32))
    for e in range(E):
        seg = srt[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg // k) > 0)
    tok_hits = np.bincount(srt // k, minlength=M)
    assert np.all(tok_hits == k)
    assert all(len(set(ids[t])) == k for t in range(M))


def test_moe_single_expert_equals_dense_bit_exact():
    M, N, O, P = 9, 16, 24, 8
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype="bf16", seed=21)
    logits = np.zeros((M, 1), np.float32)
    Y = oracle.moe_ffn(X, logits, W1[None], b1[None], W2[None], b2[None], k=1)
    assert np.array_equal(Y, oracle.ffn(X, W1, b1, W2, b2, act1=GELU))


def test_moe_identical_experts_equal_dense():
    M, N, O, P, E = 10, 16, 32, 8, 8
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype="bf16", seed=22)
    logits = np.random.default_rng(0).standard_normal((M, E)).astype(np.float32)
    st = lambda a: np.ascontiguousarray(np.broadcast_to(a, (E,) + a.shape))  # noqa: E731
    Y = oracle.moe_ffn(X, logits, st(W1), st(b1), st(W2), st(b2), k=2)
    dense = oracle.ffn(X, W1, b1, W2, b2, act1=GELU)
    np.testing.assert_allclose(Y, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


def test_moe_forced_routing_and_weighted_sum():
    M, E, N, O, P = 12, 8, 16, 24, 8
    X, logits, W1, b1, W2, b2 = synth.moe_inputs(M, E, N, O, P, seed=3,
                                                 offsets=(100, 100, 0, 0, 0, 0, 0, 0))
    ids, w, *_ = oracle.moe_route(logits, k=2)
    assert set(np.unique(ids)) == {0, 1}
    Y = oracle.moe_ffn(X, logits, W1, b1, W2, b2, k=2)
    z = [oracle.ffn(X, W1[e], b1[e], W2[e], b2[e], act1=GELU) for e in range(2)]
    for t in range(M):
        ref = w[t, 0] * z[ids[t, 0]][t] + w[t, 1] * z[ids[t, 1]][t]
        np.testing.assert_allclose(Y[t], ref, rtol=1e-14, atol=1e-14)
    assert np.all(w[:, 0] >= w[:, 1]) and np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# 7. sizes printed on the pages
# ----------------------------------------------------------------------------

def test_printed_sizes():
    g = json.load(open(os.path.join(HERE, "golden", "p1_p5_sizes.json")))
    s = g["llama3_70b_shard"]
    assert s["O"] // s["G"] == s["cols_per_gpu"]
    assert workload.shard_hidden_bytes(s["M"], s["O"], s["G"]) == s["H_shard_MiB"] * workload.MIB
    assert workload.partial_output_bytes(s["M"], s["P"]) == s["partial_Y_MiB"] * workload.MIB
    c = g["contributions"]
    assert workload.contributions_per_tile(c["O"], c["G"], c["T"]) == c["count"]
    t = g["tile_bytes"]
    assert workload.tile_bytes(t["rows"], t["cols"]) == t["KiB"] * 1024
    lb = g["largest_batch"]
    assert workload.partial_output_bytes(lb["M"], lb["implied_P"]) == lb["GiB"] * workload.GIB
    pd = g["padding"]
    assert workload.max_padding_rows(pd["W"], pd["tb_M"]) == pd["rows"]
    # the large workload is exactly that Llama 3 70B shard
    L = workload.LARGE
    assert (L.M, L.N, L.O, L.P) == (s["M"], s["N"], s["cols_per_gpu"], s["P"])


def test_flop_and_byte_counts():
    d = workload.DECODE
    assert workload.dense_flops(d.M, d.N, d.O, d.P) == 469_762_048
    assert workload.dense_bytes(d.M, d.N, d.O, d.P) == 29_634_048
    p = workload.PREFILL
    assert workload.dense_flops(p.M, p.N, p.O, p.P) == 120_259_084_288
    assert workload.dense_bytes(p.M, p.N, p.O, p.P) == 96_480_768
    t = workload.TINY_F32
    assert workload.dense_flops(t.M, t.N, t.O, t.P) == 2_097_152
    assert workload.dense_bytes(t.M, t.N, t.O, t.P, es=4) == 535_040
    m = workload.MOE
    assert workload.moe_flops(m.M * m.k, m.N, m.O, m.P) == 274_877_906_944
    assert workload.moe_bytes(m.M, m.E, m.N, m.O, m.P) == 335_773_696


# ----------------------------------------------------------------------------
# 7b. SwiGLU FFN (gated activation, no biases)
# ----------------------------------------------------------------------------

def _sigmoid_tanh_form(x):
    # sigmoid(x) = (1 + tanh(x / 2)) / 2: a different formula from 1 / (1 + e^-x)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def test_silu_pins():
    assert oracle.silu(0.0) == 0.0
    for x in np.linspace(-20, 20, 161):
        x = float(x)
        assert abs(oracle.silu(x) - x * _sigmoid_tanh_form(x)) <= 1e-15 * max(1.0, abs(x))
        # x sigmoid(x) - (-x) sigmoid(-x) = x (sigmoid(x) + sigmoid(-x)) = x
        assert abs(oracle.silu(x) - oracle.silu(-x) - x) <= 1e-14 * max(1.0, abs(x))
    assert oracle.silu(60.0) == 60.0          # gate fully open: exp(-60) is below half an ulp
    assert oracle.silu(-800.0) == 0.0         # gate shut


def test_swiglu_identity_closed_form():
    """N=O=P, Wg = 2I, Wu = Wd = I: y = silu(2x) * x = 2x^2 sigmoid(2x).  Swapping the
    gate and the up projection would give silu(x) * 2x instead."""
    n = 16
    rng = np.random.default_rng(4)
    X = rng.standard_normal((7, n)).astype(np.float32)
    eye = np.eye(n, dtype=np.float32)
    Y = oracle.swiglu(X, 2 * eye, eye, eye)
    x = X.astype(np.float64)
    expect = 2 * x * x * _sigmoid_tanh_form(2 * x)
    np.testing.assert_allclose(Y, expect, rtol=1e-14, atol=1e-300)
    swapped = 2 * x * x * _sigmoid_tanh_form(x)
    assert np.abs(Y - swapped).max() > 1e-3


def _saturated_gate_inputs(rng, M, N, O, P):
    """Dyadic inputs whose gate pre-activations are all >= 40, where silu(g) == g in
    fp64: the first input column is 8 and the first row of Wg is 8 (64 from that
    term), every other term is at most 4 in magnitude and there are at most 5 of them."""
    assert N <= 6
    X, Wg, Wu, Wd = (_dyadic(rng, s) for s in [(M, N), (N, O), (N, O), (O, P)])
    X[:, 0] = 8.0
    Wg[0, :] = 8.0
    return X, Wg, Wu, Wd


def _frac_swiglu_open_gate(X, Wg, Wu, Wd):
    """Exact Y = ((X Wg) * (X Wu)) Wd in Fractions (the gate is fully open)."""
    M, N = X.shape
    O, P = Wd.shape
    F = lambda v: Fraction(float(v))  # noqa: E731
    out = []
    for m in range(M):
        g = [sum(F(X[m, n]) * F(Wg[n, o]) for n in range(N)) for o in range(O)]
        u = [sum(F(X[m, n]) * F(Wu[n, o]) for n in range(N)) for o in range(O)]
        assert min(g) >= 40
        out.append([sum(g[o] * u[o] * F(Wd[o, p]) for o in range(O)) for p in range(P)])
    return out


@pytest.mark.parametrize("shape", [(2, 3, 4, 2), (3, 5, 7, 4), (1, 1, 1, 1), (4, 6, 3, 5)])
@pytest.mark.parametrize("as_bf16", [False, True])
def test_swiglu_open_gate_exact(shape, as_bf16):
    """With the gate open the SwiGLU FFN is bilinear and exact in fp64: every index of
    Wg, Wu, Wd and X is checked against a Fraction brute force."""
    M, N, O, P = shape
    rng = np.random.default_rng(sum(shape) * 31 + as_bf16)
    X, Wg, Wu, Wd = _saturated_gate_inputs(rng, M, N, O, P)
    exact = _frac_swiglu_open_gate(X, Wg, Wu, Wd)
    conv = _to_bf16 if as_bf16 else (lambda a: a)
    Y = oracle.swiglu(conv(X), conv(Wg), conv(Wu), conv(Wd))
    for m in range(M):
        for p in range(P):
            assert Y[m, p] == float(exact[m][p]), (m, p)


def test_swiglu_shut_gate_and_zero_input():
    rng = np.random.default_rng(8)
    M, N, O, P = 3, 4, 5, 6
    X, Wg, Wu, Wd = (_dyadic(rng, s) for s in [(M, N), (N, O), (N, O), (O, P)])
    X[:, 0] = 8.0
    Wg[:] = 0.0
    Wg[0, :] = -200.0                     # g = -1600: silu(g) == -0 in fp64
    assert np.all(oracle.swiglu(X, Wg, Wu, Wd) == 0.0)
    assert np.all(oracle.swiglu(np.zeros_like(X), Wg, Wu, Wd) == 0.0)


@pytest.mark.parametrize("G", [2, 4, 8])
def test_swiglu_tensor_parallel_invariant(G):
    """Column-split Wg and Wu, row-split Wd: the FFN is the sum of the shard outputs."""
    M, N, O, P = 6, 32, 64, 24
    X, Wg, Wu, Wd = synth.swiglu_inputs(M, N, O, P, dtype="bf16", seed=6)
    full = oracle.swiglu(X, Wg, Wu, Wd)
    w = O // G
    total = np.zeros_like(full)
    for g in range(G):
        sl = slice(g * w, (g + 1) * w)
        total += oracle.swiglu(X, np.ascontiguousarray(Wg[:, sl]), np.ascontiguousarray(Wu[:, sl]),
                               np.ascontiguousarray(Wd[sl, :]))
    np.testing.assert_allclose(total, full, rtol=1e-12, atol=1e-12 * np.abs(full).max())


def test_swiglu_rows_bit_exact():
    M, N, O, P = 10, 16, 24, 8
    X, Wg, Wu, Wd = synth.swiglu_inputs(M, N, O, P, dtype="bf16", seed=2)
    Y = oracle.swiglu(X, Wg, Wu, Wd)
    rows = [9, 0, 4]
    assert np.array_equal(oracle.swiglu(X, Wg, Wu, Wd, rows=rows), Y[rows])


# ----------------------------------------------------------------------------
# 7c. router logits (the gate network as one linear layer)
# ----------------------------------------------------------------------------

def _frac_router(X, Wr, br):
    M, N = X.shape
    E = Wr.shape[1]
    F = lambda v: Fraction(float(v))  # noqa: E731
    return [[sum(F(X[t, n]) * F(Wr[n, e]) for n in range(N)) + (F(br[e]) if br is not None else 0)
             for e in range(E)] for t in range(M)]


@pytest.mark.parametrize("shape", [(3, 5, 4), (1, 1, 1), (6, 16, 8), (2, 7, 3)])
@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("as_bf16", [False, True])
def test_router_logits_exact(shape, bias, as_bf16):
    M, N, E = shape
    rng = np.random.default_rng(sum(shape) + 7 * bias + as_bf16)
    X, Wr = _dyadic(rng, (M, N)), _dyadic(rng, (N, E))
    br = _dyadic(rng, (E,)) if bias else None
    exact = _frac_router(X, Wr, br)
    conv = _to_bf16 if as_bf16 else (lambda a: a)
    got = oracle.router_logits(conv(X), conv(Wr), br)
    for t in range(M):
        for e in range(E):
            assert got[t, e] == float(exact[t][e]), (t, e)


def test_router_identity_and_rows():
    """N = E, Wr = I: logits = X + br exactly; a row subset is bit-exact."""
    rng = np.random.default_rng(12)
    X = rng.standard_normal((9, 8)).astype(np.float32)
    br = rng.standard_normal(8).astype(np.float32)
    L = oracle.router_logits(X, np.eye(8, dtype=np.float32), br)
    assert np.array_equal(L, X.astype(np.float64) + br.astype(np.float64))
    assert np.array_equal(oracle.router_logits(X, np.eye(8, dtype=np.float32), br, rows=[8, 2]),
                          L[[8, 2]])


# ----------------------------------------------------------------------------
# 7d. backward: gradients against central differences of the forward oracle
# ----------------------------------------------------------------------------

def _bwd_inputs(rng, M, N, O, P):
    """Dyadic values (k/8, exact in fp32); b1 offset by 1/128 so that no
    pre-activation is exactly 0 (ReLU's kink: the difference quotient there is
    the mean of the two slopes, the reading of the derivative is 0)."""
    X, W1, W2, dY = (_dyadic(rng, s) for s in [(M, N), (N, O), (O, P), (M, P)])
    b1 = (_dyadic(rng, (O,)) + np.float32(1.0 / 128)).astype(np.float32)
    b2 = _dyadic(rng, (P,))
    return X, W1, b1, W2, b2, dY


def _loss(X, W1, b1, W2, b2, dY, act, lib=None):
    # L = sum(Y * dY): its gradient with respect to Y is dY
    return float(np.sum(oracle.ffn(X, W1, b1, W2, b2, act1=act, lib=lib) * dY.astype(np.float64)))


def _fd_grads(X, W1, b1, W2, b2, dY, act, lib=None, h=2.0 ** -10):
    out = []
    args = [X, W1, b1, W2, b2]
    for idx in range(5):
        base = args[idx]
        g = np.zeros(base.shape, np.float64)
        for pos in np.ndindex(base.shape):
            vals = []
            for sgn in (1, -1):
                pert = base.copy()
                pert[pos] = np.float32(base[pos] + sgn * h)     # exact: dyadic + 2^-10
                a = list(args)
                a[idx] = pert
                vals.append(_loss(*a, dY, act, lib=lib))
            g[pos] = (vals[0] - vals[1]) / (2 * h)
        out.append(g)
    return out   # dX, dW1, db1, dW2, db2


@pytest.mark.parametrize("shape", [(3, 5, 4, 6), (2, 3, 7, 4)])
@pytest.mark.parametrize("act", [NONE, RELU, GELU])
def test_backward_matches_finite_differences(shape, act):
    """Each gradient equals the central difference of the forward oracle: exactly
    (to rounding) for the piecewise-linear activations, to O(h^2) for GELU."""
    rng = np.random.default_rng(sum(shape) + act)
    X, W1, b1, W2, b2, dY = _bwd_inputs(rng, *shape)
    fd = _fd_grads(X, W1, b1, W2, b2, dY, act)
    got = oracle.ffn_backward(X, W1, b1, W2, dY, act1=act)
    tol = 1e-9 if act != GELU else 2e-5
    for name, g, f in zip(["dX", "dW1", "db1", "dW2", "db2"], got, fd):
        assert g.shape == f.shape, name
        np.testing.assert_allclose(g, f, rtol=0, atol=tol * (1 + np.abs(f).max()), err_msg=name)


def test_act_grad_pins():
    # GELU-tanh' against a central difference of GELU-tanh itself
    for x in np.linspace(-5, 5, 41):
        h = 1e-5
        fd = (oracle.act(GELU, x + h) - oracle.act(GELU, x - h)) / (2 * h)
        assert abs(oracle.act_grad(GELU, x) - fd) < 1e-8
    assert oracle.act_grad(GELU, 0.0) == 0.5
    assert oracle.act_grad(RELU, 2.0) == 1.0 and oracle.act_grad(RELU, -2.0) == 0.0
    assert oracle.act_grad(RELU, 0.0) == 0.0
    assert oracle.act_grad(NONE, -3.0) == 1.0


def test_backward_relu_identity_closed_form():
    """N = O = P, W1 = W2 = I, b1 = 0: dX = dY * [X > 0] exactly."""
    n = 12
    rng = np.random.default_rng(21)
    X = rng.standard_normal((7, n)).astype(np.float32)
    dY = rng.standard_normal((7, n)).astype(np.float32)
    eye = np.eye(n, dtype=np.float32)
    dX = oracle.ffn_backward(X, eye, np.zeros(n, np.float32), eye, dY, act1=RELU)[0]
    assert np.array_equal(dX, dY.astype(np.float64) * (X > 0))


def test_backward_subsets_bit_exact():
    M, N, O, P = 9, 16, 24, 8
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype="bf16", seed=4)
    dY = synth.f32_to_bf16_bits(np.random.default_rng(6).standard_normal((M, P)).astype(np.float32))
    full = oracle.ffn_backward(X, W1, b1, W2, dY, act1=GELU)
    rows, cols = [8, 0, 3], [23, 1, 7]
    sub = oracle.ffn_backward(X, W1, b1, W2, dY, act1=GELU, rows=rows, cols=cols)
    assert np.array_equal(sub[0], full[0][rows])
    assert np.array_equal(sub[1], full[1][:, cols])
    assert np.array_equal(sub[2], full[2][cols])
    assert np.array_equal(sub[3], full[3][cols])
    assert np.array_equal(sub[4], full[4])


# ----------------------------------------------------------------------------
# 8. planted mistakes in the oracle must be caught (CPU only)
# ----------------------------------------------------------------------------

MUTANTS = {
    "drop_b1": ("acc[o] + (b1 ? load(dtype, b1, o) : 0.0)", "acc[o]"),
    "drop_b2": ("acc[p] + (b2 ? load(dtype, b2, p) : 0.0)", "acc[p]"),
    "relu_sign": ("x > 0.0 ? x : 0.0", "x < 0.0 ? x : 0.0"),
    "gelu_const": ("0.044715 * x * x * x", "0.04715 * x * x * x"),
    "gelu_half": ("0.5 * x * (1.0 + tanh", "x * (1.0 + tanh"),
    "w1_transposed": ("load(dtype, W1, n * O + o)", "load(dtype, W1, (o % N) * O + (n % O))"),
    "w2_wrong_row": ("load(dtype, W2, o * P + p)", "load(dtype, W2, ((o + 1) % O) * P + p)"),
    "skip_last_n": ("for (int64_t n = 0; n < N; ++n)", "for (int64_t n = 0; n + 1 < N; ++n)"),
    "act2_ignored": ("yrow[p] = oracle_act(act2, a);", "yrow[p] = a;"),
    "tie_larger_index": ("l[e] > l[best]", "l[e] >= l[best]"),
    "softmax_unnormalised": ("/ denom;", ";"),
    "lists_descending": ("for (int64_t t = 0; t < M; ++t)\n                    for (int s = 0; s < k; ++s)\n                        if",
                         "for (int64_t t = M - 1; t >= 0; --t)\n                    for (int s = 0; s < k; ++s)\n                        if"),
    "moe_weight_dropped": ("y[p] += w[t * k + s] * z[p];", "y[p] += z[p];"),
    "swiglu_gate_up_swapped": ("g[o] = oracle_silu(g[o]) * u[o];", "g[o] = oracle_silu(u[o]) * g[o];"),
    "swiglu_no_silu": ("g[o] = oracle_silu(g[o]) * u[o];", "g[o] = g[o] * u[o];"),
    "silu_sign": ("x / (1.0 + exp(-x))", "x / (1.0 + exp(x))"),
    "swiglu_wg_cols_reversed": ("load(dtype, Wg, n * O + o)", "load(dtype, Wg, n * O + (O - 1 - o))"),
    "swiglu_wu_cols_reversed": ("load(dtype, Wu, n * O + o)", "load(dtype, Wu, n * O + (O - 1 - o))"),
    "swiglu_wd_cols_reversed": ("load(dtype, Wd, o * P + p)", "load(dtype, Wd, o * P + (P - 1 - p))"),
    "router_wr_cols_reversed": ("load(dtype, Wr, n * E + e)", "load(dtype, Wr, n * E + (E - 1 - e))"),
    "router_bias_dropped": ("acc + (br ? (double)br[e] : 0.0)", "acc"),
    "router_skip_first_n": ("for (int64_t n = 0; n < N; ++n)\n                acc +=",
                            "for (int64_t n = 1; n < N; ++n)\n                acc +="),
    "bwd_relu_grad": ("return x > 0.0 ? 1.0 : 0.0;", "return x > 0.0 ? 1.0 : 0.5;"),
    "bwd_gelu_grad_term": (" + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x);", ";"),
    "bwd_dx_w1_cols_reversed": ("acc += da[o] * load(dtype, W1, n * O + o);",
                                "acc += da[o] * load(dtype, W1, n * O + (O - 1 - o));"),
    "bwd_db1_skips_first_row": ("for (int64_t m = 0; m < M; ++m) acc += da[m];",
                                "for (int64_t m = 1; m < M; ++m) acc += da[m];"),
    "bwd_dw2_uses_preactivation": ("h[m] = oracle_act(act1, a);", "h[m] = a;"),
    "bwd_dx_no_act_grad": ("da[o] = bwd_dh(dtype, W2, dY, m, o, P) *\n                                oracle_act_grad(act1, bwd_a(dtype, X, W1, b1, m, o, N, O));",
                           "da[o] = bwd_dh(dtype, W2, dY, m, o, P);"),
    "bwd_dh_w2_cols_reversed": ("acc += load(dtype, dY, m * P + p) * load(dtype, W2, o * P + p);",
                                "acc += load(dtype, dY, m * P + p) * load(dtype, W2, o * P + (P - 1 - p));"),
    "swiglu_skip_first_n": ("x = load(dtype, X, m * N + n);\n        for (int64_t o = 0; o < O; ++o) {\n            g[o]",
                            "x = n ? load(dtype, X, m * N + n) : 0.0;\n        for (int64_t o = 0; o < O; ++o) {\n            g[o]"),
}


def _pin_suite(lib):
    """A fast subset of the pins above, run against a (possibly mutated) oracle build."""
    failures = []

    def check(name, fn):
        try:
            fn()
        except Exception:  # noqa: BLE001 -- a failing pin is the point
            failures.append(name)

    def brute():
        for shape, relu in [((3, 5, 7, 4), True), ((2, 3, 4, 2), False)]:
            M, N, O, P = shape
            rng = np.random.default_rng(1)
            X, W1, b1, W2, b2 = (_dyadic(rng, s) for s in [(M, N), (N, O), (O,), (O, P), (P,)])
            Y = oracle.ffn(X, W1, b1, W2, b2, act1=RELU if relu else NONE, lib=lib)
            ex = _frac_ffn(X, W1, b1, W2, b2, relu)
            assert all(Y[m, p] == float(ex[m][p]) for m in range(M) for p in range(P))

    def act2():
        rng = np.random.default_rng(7)
        X, W1, b1, W2, b2 = (_dyadic(rng, s) for s in [(3, 4), (4, 5), (5,), (5, 6), (6,)])
        ex = _frac_ffn(X, W1, b1, W2, b2, relu=True)
        Y = oracle.ffn(X, W1, b1, W2, b2, act1=RELU, act2=RELU, lib=lib)
        assert all(Y[m, p] == float(max(ex[m][p], Fraction(0))) for m in range(3) for p in range(6))

    def gelu():
        for x in np.linspace(-6, 6, 49):
            assert abs(oracle.act(GELU, x, lib=lib) - _gelu_sigmoid_form(x)) <= 1e-14 * max(1, abs(x))

    def routing():
        rng = np.random.default_rng(5)
        lg = (rng.integers(-3, 4, size=(65, 8)) * 0.5).astype(np.float32)
        ids, w, counts, offsets, srt = oracle.moe_route(lg, k=2, lib=lib)
        assert np.array_equal(ids, _independent_topk(lg, 2))
        assert np.allclose(w.sum(1), 1.0)
        assert np.array_equal(srt, np.argsort(ids.reshape(-1), kind="stable").astype(np.int32))

    def moe_combine():
        M, E, N, O, P = 6, 4, 8, 8, 8
        X, lg, W1, b1, W2, b2 = synth.moe_inputs(M, E, N, O, P, seed=3)
        ids, w, *_ = oracle.moe_route(lg, k=2)  # the unmutated build
        Y = oracle.moe_ffn(X, lg, W1, b1, W2, b2, k=2, lib=lib)
        z = [oracle.ffn(X, W1[e], b1[e], W2[e], b2[e], act1=GELU) for e in range(E)]
        for t in range(M):
            ref = w[t, 0] * z[ids[t, 0]][t] + w[t, 1] * z[ids[t, 1]][t]
            assert np.allclose(Y[t], ref, rtol=1e-13, atol=1e-13)

    def swiglu():
        for shape in [(3, 5, 7, 4), (2, 3, 4, 2)]:
            rng = np.random.default_rng(11)
            X, Wg, Wu, Wd = _saturated_gate_inputs(rng, *shape)
            exact = _frac_swiglu_open_gate(X, Wg, Wu, Wd)
            Y = oracle.swiglu(X, Wg, Wu, Wd, lib=lib)
            assert all(Y[m, p] == float(exact[m][p]) for m in range(shape[0]) for p in range(shape[3]))
        n = 8
        x = np.linspace(-3, 3, 3 * n).reshape(3, n).astype(np.float32)
        eye = np.eye(n, dtype=np.float32)
        Y = oracle.swiglu(x, 2 * eye, eye, eye, lib=lib)
        xd = x.astype(np.float64)
        assert np.allclose(Y, 2 * xd * xd * _sigmoid_tanh_form(2 * xd), rtol=1e-13, atol=0)

    def router():
        rng = np.random.default_rng(13)
        X, Wr, br = _dyadic(rng, (3, 6)), _dyadic(rng, (6, 4)), _dyadic(rng, (4,))
        exact = _frac_router(X, Wr, br)
        got = oracle.router_logits(X, Wr, br, lib=lib)
        assert all(got[t, e] == float(exact[t][e]) for t in range(3) for e in range(4))

    def backward():
        for act in (RELU, GELU):
            rng = np.random.default_rng(17 + act)
            X, W1, b1, W2, b2, dY = _bwd_inputs(rng, 2, 3, 4, 3)
            fd = _fd_grads(X, W1, b1, W2, b2, dY, act, lib=lib)
            got = oracle.ffn_backward(X, W1, b1, W2, dY, act1=act, lib=lib)
            for g, f in zip(got, fd):
                assert np.allclose(g, f, rtol=0, atol=2e-5 * (1 + np.abs(f).max()))

    for name, fn in [("brute", brute), ("act2", act2), ("gelu", gelu), ("routing", routing),
                     ("moe_combine", moe_combine), ("swiglu", swiglu), ("router", router),
                     ("backward", backward)]:
        check(name, fn)
    return failures


def test_unmutated_oracle_passes_pin_suite():
    assert _pin_suite(oracle.load()) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / f"oracle_{name}.c"
    c.write_text(mutated)
    so = tmp_path / f"liboracle_{name}.so"
    oracle.build(str(c), str(so))
    lib = oracle.load(str(so))
    assert _pin_suite(lib) != [], f"mutant {name} passed every pin"
