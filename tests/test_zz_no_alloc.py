"""ffn_forward_noalloc -- the dense FFN with the library's static device scratch as
its workspace -- against ffn_forward_ex with a caller-owned workspace, through the
C ABI.  Both run the same kernels, so the outputs must be bitwise equal; each
output also meets the oracle's rule.  Calls come in pairs, the second with a
smaller input, so the second reads a scratch that still holds the first call's
contents."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import transformer_ffn_fusion_amd as ffn
from transformer_ffn_fusion_amd import synth

from gpu_util import BF16_TOL, F32_TOL, compare, dev_bf16, dev_f32, host_f64, log

pytestmark = pytest.mark.gpu

ACT = {"relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH}


def _pair_case(shape, dtype, variant, act1, seed):
    import torch
    M, N, O, P = shape
    log(f"case noalloc {shape} {dtype} variant {variant}")
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype=dtype, seed=seed,
                                           bias_var=0.1 if dtype == "f32" else 0.02)
    to = dev_bf16 if dtype == "bf16" else dev_f32
    d = [to(a) for a in (X, W1, b1, W2, b2)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Y_ref = torch.empty((M, P), dtype=tdt, device="cuda")
    ws = ffn.workspace(ffn.ffn_workspace_size(M, N, O, P, ffn.BF16 if dtype == "bf16" else ffn.F32,
                                              variant))
    ffn.ffn_forward_ex(*d, Y_ref, act1, "none", variant, ws)
    Y = torch.full((M, P), float("nan"), dtype=tdt, device="cuda")
    ffn.ffn_forward_noalloc(*d, Y, act1, "none", variant)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_ref), "ffn_forward_noalloc differs from ffn_forward_ex"
    ref = oracle.ffn(X, W1, b1, W2, b2, act1=ACT[act1])
    compare(host_f64(Y), ref, BF16_TOL if dtype == "bf16" else F32_TOL, f"noalloc {shape}")


@pytest.mark.parametrize("pair", [
    # decode layers (skinny): the decode shard, then a smaller call
    [((16, 4096, 1792, 4096), "bf16", ffn.VARIANT_AUTO, "gelu_tanh", 0),
     ((5, 1024, 512, 264), "bf16", ffn.VARIANT_AUTO, "gelu_tanh", 1)],
    # fused kernel + ordered reduce: split partials in the scratch
    [((200, 512, 1792, 1032), "bf16", ffn.VARIANT_FUSED, "gelu_tanh", 2),
     ((70, 264, 456, 520), "bf16", ffn.VARIANT_FUSED, "relu", 3)],
    # fp32 path: the tiny workload, then a smaller one
    [((8, 128, 512, 128), "f32", ffn.VARIANT_AUTO, "relu", 4),
     ((3, 40, 520, 72), "f32", ffn.VARIANT_AUTO, "relu", 5)],
])
def test_noalloc_matches_workspace_call(pair):
    for case in pair:
        _pair_case(*case)


def test_noalloc_refuses_oversized_shape_and_leaves_output_untouched():
    import torch
    M, N, O, P = 4096, 64, 1792, 512     # 24 MiB of split partials
    assert ffn.ffn_workspace_size(M, N, O, P) > ffn.NOALLOC_SCRATCH_BYTES
    X, W1, b1, W2, b2 = (dev_bf16(a) for a in synth.dense_inputs(M, N, O, P, seed=6))
    Y = torch.full((M, P), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ffn.FFNError, match="static scratch"):
        ffn.ffn_forward_noalloc(X, W1, b1, W2, b2, Y)
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())
