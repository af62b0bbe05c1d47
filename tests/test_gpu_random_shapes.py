"""Seeded random shapes through every forward kernel family, against the fp64 oracle.

The fixed shape lists of the other parity tests pick tails by hand; this sweep
draws them: M from 1 to 300 rows, N, O, P multiples of 8 up to ~1.5k (so every
partial row tile, k tail, ragged hidden chunk and ragged output pass is hit in
some case), random activations and bias presence, and MoE layers with random
expert counts and top-k.  Shapes and seeds come from numpy's PCG64 with a
fixed seed, so every run checks the same cases, and each case is logged before
it runs.

Rule: the plain bf16 rule, max |Y - Yref| <= 2e-2 rms(Yref), wherever the
exact output's own rounding to bf16 leaves room for it.  Random layers can
have heavier-tailed outputs than the workloads (a top-5 average of narrow
experts reaches max|Y| = 6.1 rms): rounding the exact Y alone then moves its
largest element, just above a power of two, by 2^-8 |y| = 2.07e-2 rms, beyond
the rule whatever computes it.  Where that floor exceeds 1.6e-2 rms the
check allows one bf16 rounding per element instead (|Y - Yref| <=
2e-2 rms + 2^-8 |Yref|).  The workload tests use the plain rule only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import transformer_ffn_fusion_amd as ffn
from transformer_ffn_fusion_amd import synth

from gpu_util import (BF16_TOL, compare, compare_with_bf16_rounding, dev_bf16, dev_f32,
                      host_f64, log)

pytestmark = pytest.mark.gpu

ACTS = ("relu", "gelu_tanh", "none")
ACT_CODE = {"relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH, "none": oracle.ACT_NONE}


def _check(got, ref, what):
    """The plain rule, or one bf16 rounding per element where the exact output's
    own rounding floor leaves no room for the plain rule (see the module text)."""
    from transformer_ffn_fusion_amd import synth
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rounded = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(ref.astype(np.float32)))
    floor = float(np.max(np.abs(rounded.astype(np.float64) - ref))) / max(rms, 1e-30)
    if floor < 1.6e-2:
        compare(got, ref, BF16_TOL, what)
    else:
        log(f"  {what}: rounding the exact output alone costs {floor:.3e} rms")
        compare_with_bf16_rounding(got, ref, BF16_TOL, what)


def _dense_cases(n=16):
    rng = np.random.default_rng(2024)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 301))
        N, O, P = (8 * int(rng.integers(1, 192)) for _ in range(3))
        out.append((M, N, O, P, ACTS[int(rng.integers(0, 3))], bool(rng.integers(0, 2)), 100 + i))
    return out


@pytest.mark.parametrize("M,N,O,P,act1,bias,seed", _dense_cases())
@pytest.mark.parametrize("variant", [ffn.VARIANT_AUTO, ffn.VARIANT_FUSED])
def test_random_dense(M, N, O, P, act1, bias, seed, variant):
    import torch
    if variant == ffn.VARIANT_AUTO and M > 16:
        M = 1 + M % 16          # the automatic choice at these row counts is the decode form
    log(f"case random dense {(M, N, O, P)} act1={act1} bias={bias} variant={variant}")
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, seed=seed, with_bias=bias)
    d = [None if a is None else dev_bf16(a) for a in (X, W1, b1, W2, b2)]
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    ffn.ffn_forward_ex(*d, Y, act1, "none", variant)
    torch.cuda.synchronize()
    ref = oracle.ffn(X, W1, b1, W2, b2, act1=ACT_CODE[act1], act2=oracle.ACT_NONE)
    _check(host_f64(Y), ref, f"random dense {(M, N, O, P)}")


def _decode_stream_cases(n=8):
    # the decode stream's shape family: M 1..16, N = P = 4096, O a multiple of 256 up to 2048
    rng = np.random.default_rng(4096)
    return [(int(rng.integers(1, 17)), 4096, 256 * int(rng.integers(1, 9)), 4096,
             ACTS[int(rng.integers(0, 3))], ACTS[int(rng.integers(0, 3))], bool(rng.integers(0, 2)),
             bool(rng.integers(0, 2)), 500 + i) for i in range(n)]


@pytest.mark.parametrize("M,N,O,P,act1,act2,bias,gated,seed", _decode_stream_cases())
def test_random_decode_stream(M, N, O, P, act1, act2, bias, gated, seed):
    import torch
    log(f"case random decode stream {(M, N, O, P)} act1={act1} act2={act2} bias={bias} "
        f"gated={gated}")
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    if gated:
        X, Wg, Wu, Wd = synth.swiglu_inputs(M, N, O, P, seed=seed)
        ffn.ffn_swiglu_forward(*(dev_bf16(a) for a in (X, Wg, Wu, Wd)), Y, ffn.VARIANT_DECODE)
        torch.cuda.synchronize()
        ref = oracle.swiglu(X, Wg, Wu, Wd)
    else:
        X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, seed=seed, with_bias=bias)
        d = [None if a is None else dev_bf16(a) for a in (X, W1, b1, W2, b2)]
        ffn.ffn_forward_ex(*d, Y, act1, act2, ffn.VARIANT_DECODE)
        torch.cuda.synchronize()
        ref = oracle.ffn(X, W1, b1, W2, b2, act1=ACT_CODE[act1], act2=ACT_CODE[act2])
    _check(host_f64(Y), ref, f"random decode stream {(M, N, O, P)}")


def _swiglu_cases(n=8):
    rng = np.random.default_rng(77)
    return [(int(rng.integers(1, 200)), *(8 * int(rng.integers(1, 160)) for _ in range(3)), 300 + i)
            for i in range(n)]


@pytest.mark.parametrize("M,N,O,P,seed", _swiglu_cases())
def test_random_swiglu(M, N, O, P, seed):
    import torch
    log(f"case random swiglu {(M, N, O, P)}")
    X, Wg, Wu, Wd = synth.swiglu_inputs(M, N, O, P, seed=seed)
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    ffn.ffn_swiglu_forward(*(dev_bf16(a) for a in (X, Wg, Wu, Wd)), Y)
    torch.cuda.synchronize()
    _check(host_f64(Y), oracle.swiglu(X, Wg, Wu, Wd), f"random swiglu {(M, N, O, P)}")


def _moe_cases(n=8):
    rng = np.random.default_rng(4242)
    out = []
    for i in range(n):
        E = int(rng.choice([2, 3, 8, 16, 33]))
        k = int(rng.integers(1, min(E, 8) + 1))
        M = int(rng.integers(1, 400))
        N, O, P = (8 * int(rng.integers(1, 96)) for _ in range(3))
        out.append((M, E, k, N, O, P, 500 + i))
    return out


@pytest.mark.parametrize("M,E,k,N,O,P,seed", _moe_cases())
def test_random_moe(M, E, k, N, O, P, seed):
    import torch
    log(f"case random moe M={M} E={E} k={k} {(N, O, P)}")
    X, logits, W1, b1, W2, b2 = synth.moe_inputs(M, E, N, O, P, seed=seed,
                                                 offsets=tuple(np.linspace(0.6, -0.6, E)))
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    ffn.moe_ffn_forward(dev_bf16(X), dev_f32(logits), k, dev_bf16(W1), dev_bf16(b1), dev_bf16(W2),
                        dev_bf16(b2), Y, topk_ids=ids)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), oracle.moe_route(logits, k=k)[0])
    ref = oracle.moe_ffn(X, logits, W1, b1, W2, b2, k=k)
    _check(host_f64(Y), ref, f"random moe M={M} E={E} k={k}")
