"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module generates inputs only.  It holds none of the feed-forward
arithmetic: no activation, no bias addition, no FFN or router product and no
routing.
Both sides of every parity check (the HIP library and the fp64 oracle) receive
the arrays produced here, bit for bit.

Recipe (seeds, drawing order and the variance reading are choices of this package):
* ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal(dtype=float32)``
  scaled by the standard deviation, in the order X, W1, b1, W2, b2
  (MoE with logits as input: X, the logit draws, then per expert W1_e, b1_e,
  W2_e, b2_e; MoE with the router: X, Wr, then the experts);
* standard deviations: X 1, W1 1/sqrt(N), W2 1/sqrt(O), Wr 1/sqrt(N), biases
  sqrt(v) with v read as a variance (0.1 for the tiny fp32 case, 0.02 else);
* bf16 tensors are the fp32 draws rounded once to nearest, ties to even;
* MoE gate logits, where they are an input of the layer, are drawn directly:
  a standard normal draw (the spread of a unit-variance token through a
  1/sqrt(N)-scaled router) plus the per-expert offset, rounded once to fp32;
  where the router runs on the GPU its weights Wr (bf16) and the offsets as
  its bias br (fp32) are the inputs instead.
"""
from __future__ import annotations

import numpy as np

# Per-expert logit offsets that skew the expert load (from the MoE workload spec).
MOE_SKEW_OFFSETS = (0.8, 0.4, 0.2, 0.0, 0.0, -0.2, -0.4, -0.8)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Adding 0x7FFF plus the lowest kept bit and truncating is round-to-nearest-even
    on the 16 dropped bits; it cannot overflow 32 bits for finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if not np.all(np.isfinite(x)):
        raise ValueError("only finite values are generated")
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng, shape, std):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def dense_inputs(M, N, O, P, *, dtype="bf16", bias_var=0.02, seed=0, with_bias=True):
    """X (MxN), W1 (NxO), b1 (O), W2 (OxP), b2 (P).

    ``dtype="bf16"`` returns uint16 bf16 bit patterns, ``"f32"`` float32 arrays."""
    rng = np.random.default_rng(seed)
    X = _draw(rng, (M, N), 1.0)
    W1 = _draw(rng, (N, O), 1.0 / np.sqrt(N))
    b1 = _draw(rng, (O,), np.sqrt(bias_var))
    W2 = _draw(rng, (O, P), 1.0 / np.sqrt(O))
    b2 = _draw(rng, (P,), np.sqrt(bias_var))
    if not with_bias:
        b1 = b2 = None
    out = (X, W1, b1, W2, b2)
    if dtype == "bf16":
        out = tuple(None if a is None else f32_to_bf16_bits(a) for a in out)
    elif dtype != "f32":
        raise ValueError(dtype)
    return out


def swiglu_inputs(M, N, O, P, *, dtype="bf16", seed=0):
    """X (MxN), Wg and Wu (NxO), Wd (OxP) for the SwiGLU FFN (no biases); the same
    Gaussian scaling as dense_inputs (unit-variance X, 1/sqrt(fan_in) weights)."""
    rng = np.random.default_rng(seed)
    X = _draw(rng, (M, N), 1.0)
    Wg = _draw(rng, (N, O), 1.0 / np.sqrt(N))
    Wu = _draw(rng, (N, O), 1.0 / np.sqrt(N))
    Wd = _draw(rng, (O, P), 1.0 / np.sqrt(O))
    out = (X, Wg, Wu, Wd)
    if dtype == "bf16":
        out = tuple(f32_to_bf16_bits(a) for a in out)
    elif dtype != "f32":
        raise ValueError(dtype)
    return out


def _offsets(offsets, E):
    return np.asarray(offsets[:E] if len(offsets) >= E else list(offsets) + [0.0] * (E - len(offsets)),
                      dtype=np.float64)


def _experts(rng, E, N, O, P, bias_var):
    W1 = np.empty((E, N, O), np.uint16)
    b1 = np.empty((E, O), np.uint16)
    W2 = np.empty((E, O, P), np.uint16)
    b2 = np.empty((E, P), np.uint16)
    for e in range(E):
        W1[e] = f32_to_bf16_bits(_draw(rng, (N, O), 1.0 / np.sqrt(N)))
        b1[e] = f32_to_bf16_bits(_draw(rng, (O,), np.sqrt(bias_var)))
        W2[e] = f32_to_bf16_bits(_draw(rng, (O, P), 1.0 / np.sqrt(O)))
        b2[e] = f32_to_bf16_bits(_draw(rng, (P,), np.sqrt(bias_var)))
    return W1, b1, W2, b2


def moe_inputs(M, E, N, O, P, *, offsets=MOE_SKEW_OFFSETS, bias_var=0.02, seed=0):
    """bf16 MoE inputs with the gate logits given: X (MxN), logits (MxE, fp32), W1 (ExNxO),
    b1 (ExO), W2 (ExOxP), b2 (ExP)."""
    rng = np.random.default_rng(seed)
    X = f32_to_bf16_bits(_draw(rng, (M, N), 1.0))
    noise = _draw(rng, (M, E), 1.0)
    W1, b1, W2, b2 = _experts(rng, E, N, O, P, bias_var)
    logits = (noise.astype(np.float64) + _offsets(offsets, E)).astype(np.float32)
    return X, logits, W1, b1, W2, b2


def moe_router_inputs(M, E, N, O, P, *, offsets=MOE_SKEW_OFFSETS, bias_var=0.02, seed=0):
    """bf16 MoE inputs with the router on the GPU: X (MxN), Wr (NxE bf16, std 1/sqrt(N)),
    br (E fp32: the per-expert offsets), W1, b1, W2, b2 as in moe_inputs."""
    rng = np.random.default_rng(seed)
    X = f32_to_bf16_bits(_draw(rng, (M, N), 1.0))
    Wr = f32_to_bf16_bits(_draw(rng, (N, E), 1.0 / np.sqrt(N)))
    W1, b1, W2, b2 = _experts(rng, E, N, O, P, bias_var)
    br = _offsets(offsets, E).astype(np.float32)
    return X, Wr, br, W1, b1, W2, b2


def check_rows(M, block=64, n_random=249, seed=1):
    """Rows checked at full size: tile edges, the middle, the tail, plus random rows."""
    fixed = {0, 1, block - 1, block, M // 2, M - 2, M - 1}
    fixed = {r for r in fixed if 0 <= r < M}
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(M), np.fromiter(fixed, dtype=np.int64))
    extra = rng.choice(pool, size=min(n_random, pool.size), replace=False) if pool.size else []
    return np.array(sorted(fixed | set(int(r) for r in extra)), dtype=np.int64)
