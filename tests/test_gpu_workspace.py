"""The workspace holds per-call intermediates only and needs no initialisation:
every entry point reads only workspace bytes that the same call wrote before.
A call on a workspace filled with 0xFF bytes (NaN for every fp32 slot, -1 for
every index slot) must give the same bits as a call on a zeroed workspace."""
from __future__ import annotations

import numpy as np
import pytest

import transformer_ffn_fusion_amd as ffn
from transformer_ffn_fusion_amd import synth

from gpu_util import dev_bf16, dev_f32, log

pytestmark = pytest.mark.gpu


def _twice(run, ws):
    """Outputs of run(ws) on a zeroed workspace, then on one filled with 0xFF."""
    import torch
    ws.zero_()
    first = [t.clone() for t in run(ws)]
    torch.cuda.synchronize()
    ws.fill_(255)
    second = run(ws)
    torch.cuda.synchronize()
    return first, second


def _dense(M, N, O, P):
    import torch
    X, W1, b1, W2, b2 = (dev_bf16(a) for a in synth.dense_inputs(M, N, O, P, seed=3))
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")

    def run(ws):
        ffn.ffn_forward(X, W1, b1, W2, b2, Y, ws=ws)
        return [Y]
    return run, ffn.workspace(ffn.ffn_workspace_size(M, N, O, P))


def _swiglu(M, N, O, P):
    import torch
    X, Wg, Wu, Wd = (dev_bf16(a) for a in synth.swiglu_inputs(M, N, O, P, seed=4))
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")

    def run(ws):
        ffn.ffn_swiglu_forward(X, Wg, Wu, Wd, Y, ws=ws)
        return [Y]
    return run, ffn.workspace(ffn.ffn_swiglu_workspace_size(M, N, O, P))


def _moe(M, E, k, N, O, P):
    import torch
    X, lg, W1, b1, W2, b2 = synth.moe_inputs(M, E, N, O, P, seed=5)
    X, W1, b1, W2, b2 = (dev_bf16(a) for a in (X, W1, b1, W2, b2))
    lg = dev_f32(lg)
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    srt = torch.empty(M * k, dtype=torch.int32, device="cuda")

    def run(ws):
        ffn.moe_ffn_forward(X, lg, k, W1, b1, W2, b2, Y, topk_ids=ids, sorted_entries=srt, ws=ws)
        return [Y, ids, srt]
    return run, ffn.workspace(ffn.moe_workspace_size(M, E, k, N, O, P))


def _backward(M, N, O, P):
    import torch
    X, W1, b1, W2, _ = (dev_bf16(a) if a is not None else None
                        for a in synth.dense_inputs(M, N, O, P, seed=6))
    dY = dev_bf16(synth.f32_to_bf16_bits(
        np.random.default_rng(7).standard_normal((M, P)).astype(np.float32)))
    dX = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dW1 = torch.empty((N, O), dtype=torch.float32, device="cuda")
    db1 = torch.empty(O, dtype=torch.float32, device="cuda")
    dW2 = torch.empty((O, P), dtype=torch.float32, device="cuda")
    db2 = torch.empty(P, dtype=torch.float32, device="cuda")

    def run(ws):
        ffn.ffn_backward(X, W1, b1, W2, dY, dX, dW1, db1, dW2, db2, ws=ws)
        return [dX, dW1, db1, dW2, db2]
    return run, ffn.workspace(ffn.ffn_backward_workspace_size(M, N, O, P))


CASES = {
    "fused, 4 splits, ragged tiles": lambda: _dense(130, 512, 1792, 1032),
    "decode, split K": lambda: _dense(16, 1000, 904, 520),
    "swiglu": lambda: _swiglu(130, 256, 1024, 264),
    "swiglu decode": lambda: _swiglu(5, 512, 448, 136),
    "moe top-2": lambda: _moe(300, 8, 2, 64, 1024, 2048),
    "moe, many experts": lambda: _moe(200, 64, 3, 64, 448, 128),
    "backward": lambda: _backward(130, 264, 456, 136),
}


@pytest.mark.parametrize("name", list(CASES))
def test_workspace_needs_no_initialisation(name):
    import torch
    log(f"case workspace contents: {name}")
    run, ws = CASES[name]()
    first, second = _twice(run, ws)
    for a, b in zip(first, second):
        assert bool(torch.isfinite(a.float()).all()) if a.is_floating_point() else True
        assert torch.equal(a, b), f"{name}: output depends on the workspace's prior contents"
