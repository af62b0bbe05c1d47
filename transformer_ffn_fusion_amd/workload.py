"""Workload definitions and algorithmic work counts (no arithmetic of the method).

The five workloads are the shapes the fused feed-forward path is measured and
checked on.  Dense shapes are (M tokens, N input width, O hidden width of one
tensor-parallel shard, P output width); the hidden widths 1792 and 3584 are
1/8 shards of 14,336 and 28,672 (the kernel-fusion / tensor-parallelism post,
brunomaga.github.io, sections "Megatron-LM tensor parallelism" and "Results").

Algorithmic FLOPs are 2*M*(N*O + O*P); algorithmic bytes are what the
computation must move at minimum: its external inputs and outputs (the
kernel-fusion explainer, tirogla.com, "How it works": a fused chain costs the
HBM bytes of its external inputs and outputs).  Workspace, partial sums and
re-reads are not counted.
"""
from __future__ import annotations

from dataclasses import dataclass

MIB = 1 << 20
GIB = 1 << 30


@dataclass(frozen=True)
class Dense:
    name: str
    M: int
    N: int
    O: int
    P: int
    dtype: str          # "bf16" or "f32"
    act1: str           # "relu" or "gelu_tanh"
    bias_var: float


@dataclass(frozen=True)
class MoE:
    name: str
    M: int
    E: int
    k: int
    N: int
    O: int
    P: int
    dtype: str
    act1: str
    bias_var: float


TINY_F32 = Dense("tiny_fp32_8x128x512x128", 8, 128, 512, 128, "f32", "relu", 0.1)
DECODE = Dense("decode_shard_16x4096x1792x4096", 16, 4096, 1792, 4096, "bf16", "gelu_tanh", 0.02)
PREFILL = Dense("prefill_shard_4096x4096x1792x4096", 4096, 4096, 1792, 4096, "bf16", "gelu_tanh", 0.02)
LARGE = Dense("large_shard_8192x8192x3584x8192", 8192, 8192, 3584, 8192, "bf16", "gelu_tanh", 0.02)
MOE = MoE("moe_top2_4096tok_8x4096x2048x4096", 4096, 8, 2, 4096, 2048, 4096, "bf16", "gelu_tanh", 0.02)

ALL = (TINY_F32, DECODE, PREFILL, LARGE, MOE)

# One GPU's share of the same MoE layer sharded 8 ways over the hidden width of
# every expert (2048 / 8 = 256 per expert; the kernel-fusion post, section
# "Results": expert sharding keeps all experts on every GPU with O/G columns).
MOE_SHARD = MoE("moe_top2_4096tok_8x4096x256x4096_expert_shard", 4096, 8, 2, 4096, 256, 4096,
                "bf16", "gelu_tanh", 0.02)


@dataclass(frozen=True)
class Gated:
    """A SwiGLU FFN shard: (silu(X Wg) * (X Wu)) Wd, no biases (the kernel-fusion
    post, section "Benchmarks": the benchmarked models are SwiGLU models)."""
    name: str
    M: int
    N: int
    O: int
    P: int
    dtype: str


# the same one-GPU shard as PREFILL/DECODE (1792 = 14,336 / 8), with the gated FFN
SWIGLU_PREFILL = Gated("swiglu_prefill_shard_4096x4096x1792x4096", 4096, 4096, 1792, 4096, "bf16")
SWIGLU_DECODE = Gated("swiglu_decode_shard_16x4096x1792x4096", 16, 4096, 1792, 4096, "bf16")


def esize(dtype: str) -> int:
    return 2 if dtype == "bf16" else 4


def dense_flops(M, N, O, P) -> int:
    return 2 * M * (N * O + O * P)


def dense_bytes(M, N, O, P, es=2, bias=True) -> int:
    """X + W1 + b1 + W2 + b2 + Y."""
    b = (O + P) if bias else 0
    return es * (M * N + N * O + O * P + M * P + b)


def swiglu_flops(M, N, O, P) -> int:
    """Two N x O products (gate and up) and one O x P product per row."""
    return 2 * M * (2 * N * O + O * P)


def swiglu_bytes(M, N, O, P, es=2) -> int:
    """X + Wg + Wu + Wd + Y."""
    return es * (M * N + 2 * N * O + O * P + M * P)


def moe_flops(rows, N, O, P) -> int:
    """Counted over the real (token, expert) rows; padding rows are not counted."""
    return 2 * rows * (N * O + O * P)


def moe_bytes(M, E, N, O, P, es=2) -> int:
    """X + fp32 logits + every expert's weights and biases + Y."""
    return es * (M * N + E * (N * O + O + O * P + P) + M * P) + 4 * M * E


def shard_hidden_bytes(M, O_total, G, es=2) -> int:
    """Bytes of one shard's hidden activations H^(g): M x (O/G)."""
    return M * (O_total // G) * es


def partial_output_bytes(M, P, es=2) -> int:
    """Bytes of one shard's partial output H^(g) W2^(g): M x P."""
    return M * P * es


def contributions_per_tile(O_total, G, T) -> int:
    """Hidden-dimension tiles of width T contributing to one output tile: ceil((O/G)/T)."""
    return -(-(O_total // G) // T)


def tile_bytes(rows, cols, es=2) -> int:
    return rows * cols * es


def max_padding_rows(W, tb_m) -> int:
    """Worst-case zero rows added when W row groups are each padded to a multiple of tb_m."""
    return (W - 1) * (tb_m - 1)
