"""The five workload definitions and the input recipe, pinned on the CPU.

The workloads are fixed data: a change to a shape, an activation, a variance
or the MoE logit offsets changes what every parity test and the bench
measure, so each is written out here once more and compared.  The recipe
checks draw small tensors with the same generator calls as the full-size
workloads and compare their sample moments with the stated distributions.
"""
import numpy as np
import pytest

from transformer_ffn_fusion_amd import synth, workload


def test_the_five_workloads():
    want = {
        # name: (M, N, O, P, dtype, act1, bias variance)
        "tiny_fp32_8x128x512x128": (8, 128, 512, 128, "f32", "relu", 0.1),
        "decode_shard_16x4096x1792x4096": (16, 4096, 1792, 4096, "bf16", "gelu_tanh", 0.02),
        "prefill_shard_4096x4096x1792x4096": (4096, 4096, 1792, 4096, "bf16", "gelu_tanh", 0.02),
        "large_shard_8192x8192x3584x8192": (8192, 8192, 3584, 8192, "bf16", "gelu_tanh", 0.02),
    }
    dense = [c for c in workload.ALL if isinstance(c, workload.Dense)]
    assert {c.name for c in dense} == set(want)
    for c in dense:
        assert (c.M, c.N, c.O, c.P, c.dtype, c.act1, c.bias_var) == want[c.name], c.name
    moe = [c for c in workload.ALL if isinstance(c, workload.MoE)]
    assert len(moe) == 1 and len(workload.ALL) == 5
    m = moe[0]
    assert (m.M, m.E, m.k, m.N, m.O, m.P, m.dtype, m.act1, m.bias_var) == \
        (4096, 8, 2, 4096, 2048, 4096, "bf16", "gelu_tanh", 0.02)
    assert synth.MOE_SKEW_OFFSETS == (0.8, 0.4, 0.2, 0.0, 0.0, -0.2, -0.4, -0.8)


def test_shard_widths_are_one_eighth():
    # 1792 and 3584 are 1/8 of the 14,336- and 28,672-wide hidden layers;
    # the expert-sharded share is 1/8 of an expert's 2048
    assert workload.DECODE.O * 8 == 14336 and workload.PREFILL.O * 8 == 14336
    assert workload.LARGE.O * 8 == 28672
    assert workload.MOE_SHARD.O * 8 == workload.MOE.O
    s, m = workload.MOE_SHARD, workload.MOE
    assert (s.M, s.E, s.k, s.N, s.P) == (m.M, m.E, m.k, m.N, m.P)


def _std(a_bits_or_f32, bf16):
    a = synth.bf16_bits_to_f32(a_bits_or_f32) if bf16 else a_bits_or_f32
    return float(np.std(a.astype(np.float64))), float(np.mean(a.astype(np.float64)))


@pytest.mark.parametrize("dtype,bias_var", [("bf16", 0.02), ("f32", 0.1)])
def test_dense_recipe_moments(dtype, bias_var):
    M, N, O, P = 256, 512, 384, 640
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype=dtype, bias_var=bias_var, seed=3)
    bf = dtype == "bf16"
    for a, std, n in ((X, 1.0, M * N), (W1, 1 / np.sqrt(N), N * O), (W2, 1 / np.sqrt(O), O * P),
                      (b1, np.sqrt(bias_var), O), (b2, np.sqrt(bias_var), P)):
        s, mu = _std(a, bf)
        # sample std and mean of n normal draws: relative error ~ 1/sqrt(2n), mean ~ std/sqrt(n)
        assert abs(s / std - 1) < 6 / np.sqrt(2 * n), (s, std)
        assert abs(mu) < 6 * std / np.sqrt(n), (mu, std)
    if bf:
        assert X.dtype == np.uint16 and W1.dtype == np.uint16
    else:
        assert X.dtype == np.float32


def test_moe_recipe_offsets_and_router_bias():
    M, E, N, O, P = 2048, 8, 256, 64, 128
    X, logits, W1, b1, W2, b2 = synth.moe_inputs(M, E, N, O, P, seed=5)
    assert logits.dtype == np.float32 and logits.shape == (M, E)
    # per-expert mean of the drawn logits is the offset (unit-variance draws)
    mu = logits.astype(np.float64).mean(axis=0)
    assert np.all(np.abs(mu - np.asarray(synth.MOE_SKEW_OFFSETS)) < 6 / np.sqrt(M))
    Xr, Wr, br, *_ = synth.moe_router_inputs(M, E, N, O, P, seed=5)
    assert br.dtype == np.float32 and tuple(float(v) for v in br) == \
        tuple(float(np.float32(v)) for v in synth.MOE_SKEW_OFFSETS)
    s, _ = _std(Wr, True)
    assert abs(s * np.sqrt(N) - 1) < 6 / np.sqrt(2 * N * E)
