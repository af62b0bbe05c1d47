"""GPU parity of the SwiGLU FFN (silu(X Wg) * (X Wu)) Wd, through the C ABI, against
the fp64 oracle.  Same tolerance rule as the dense tests: max |Y - Yref| <= 2e-2 *
rms(Yref) for bf16 data with fp32 accumulation, <= 1e-5 * rms(Yref) for fp32."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import transformer_ffn_fusion_amd as ffn
from transformer_ffn_fusion_amd import synth, workload

from gpu_util import BF16_TOL, F32_TOL, compare, dev_bf16, dev_f32, host_f64, log

pytestmark = pytest.mark.gpu


def _run(M, N, O, P, *, dtype="bf16", variant=0, seed=0, rows=None, repeat=1):
    import torch
    X, Wg, Wu, Wd = synth.swiglu_inputs(M, N, O, P, dtype=dtype, seed=seed)
    to = dev_bf16 if dtype == "bf16" else dev_f32
    dX, dWg, dWu, dWd = to(X), to(Wg), to(Wu), to(Wd)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Y = torch.empty((M, P), dtype=tdt, device="cuda")
    code = ffn.BF16 if dtype == "bf16" else ffn.F32
    ws = ffn.workspace(ffn.ffn_swiglu_workspace_size(M, N, O, P, code, variant))
    outs = []
    for _ in range(repeat):
        ffn.ffn_swiglu_forward(dX, dWg, dWu, dWd, Y, variant, ws)
        torch.cuda.synchronize()
        outs.append(Y.clone())
    ref = oracle.swiglu(X, Wg, Wu, Wd, rows=rows)
    got = host_f64(Y if rows is None else Y[torch.as_tensor(rows, device="cuda")])
    return got, ref, outs


@pytest.mark.parametrize("shape", [
    (1, 64, 256, 512),       # one row, one 256-column chunk (one pass), one output pass
    (65, 264, 456, 520),     # two-pass chunks of 448: the second holds 8 columns (pass B empty)
    (130, 512, 1792, 1032),  # 4 two-pass chunks of 448, 3 row tiles (last ragged)
    (96, 192, 896, 520),     # 2 two-pass chunks, ragged output pass
    (200, 128, 1024, 64),    # 4 one-pass chunks of 256, narrow output
    (64, 1000, 904, 1544),   # ragged everywhere: chunks 448, 448, 8
    (33, 96, 2048, 256),     # 8 one-pass chunks of 256
])
def test_swiglu_fused_shapes(shape):
    M, N, O, P = shape
    log(f"case swiglu fused {shape}")
    got, ref, _ = _run(M, N, O, P, variant=ffn.VARIANT_FUSED, seed=M + N)
    compare(got, ref, BF16_TOL, f"swiglu fused {shape}")


@pytest.mark.parametrize("shape", [
    (1, 256, 128, 128),
    (5, 200, 264, 136),       # one K block (the gated layer still writes partials)
    (7, 520, 264, 136),       # ragged K blocks and column blocks
    (16, 1024, 3584, 512),
])
def test_swiglu_skinny_shapes(shape):
    M, N, O, P = shape
    log(f"case swiglu skinny {shape}")
    got, ref, _ = _run(M, N, O, P, variant=ffn.VARIANT_SKINNY, seed=M * 7 + P)
    compare(got, ref, BF16_TOL, f"swiglu skinny {shape}")


@pytest.mark.parametrize("shape", [(3, 40, 520, 72), (37, 136, 264, 264)])
def test_swiglu_fp32_shapes(shape):
    M, N, O, P = shape
    log(f"case swiglu fp32 {shape}")
    got, ref, _ = _run(M, N, O, P, dtype="f32", seed=M + 1)
    compare(got, ref, F32_TOL, f"swiglu fp32 {shape}")


def test_swiglu_fused_and_skinny_agree_at_m16():
    M, N, O, P = 16, 1024, 896, 1024
    log("case swiglu fused vs skinny at M=16")
    a, ref, _ = _run(M, N, O, P, variant=ffn.VARIANT_FUSED, seed=3)
    b, _, _ = _run(M, N, O, P, variant=ffn.VARIANT_SKINNY, seed=3)
    compare(a, ref, BF16_TOL, "fused")
    compare(b, ref, BF16_TOL, "skinny")


def test_swiglu_tensor_parallel_shards():
    """Four shards (columns of Wg and Wu, rows of Wd) summed in fp64 equal the full FFN."""
    import torch
    M, N, O, P = 96, 256, 1024, 512
    X, Wg, Wu, Wd = synth.swiglu_inputs(M, N, O, P, seed=12)
    ref = oracle.swiglu(X, Wg, Wu, Wd)
    total = np.zeros_like(ref)
    w = O // 4
    log("case swiglu 4 shards")
    for g in range(4):
        sl = slice(g * w, (g + 1) * w)
        Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
        ffn.ffn_swiglu_forward(dev_bf16(X), dev_bf16(np.ascontiguousarray(Wg[:, sl])),
                               dev_bf16(np.ascontiguousarray(Wu[:, sl])),
                               dev_bf16(np.ascontiguousarray(Wd[sl, :])), Y)
        torch.cuda.synchronize()
        total += host_f64(Y)
    compare(total, ref, BF16_TOL, "sum of 4 shards")


def test_swiglu_zero_rows_and_errors():
    import torch
    dX = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    dW = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    dWd = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = ffn.workspace(ffn.ffn_swiglu_workspace_size(4, 64, 256, 64))
    L = ffn.lib()
    # M == 0: nothing written
    rc = L.ffn_swiglu_forward(dX.data_ptr(), dW.data_ptr(), dW.data_ptr(), dWd.data_ptr(),
                              Y.data_ptr(), 0, 64, 256, 64, ffn.BF16, 0, ws.data_ptr(), ws.numel(), None)
    assert rc == 0
    # missing Wu, short workspace: rejected before launch, Y untouched
    rc = L.ffn_swiglu_forward(dX.data_ptr(), dW.data_ptr(), None, dWd.data_ptr(), Y.data_ptr(),
                              4, 64, 256, 64, ffn.BF16, 0, ws.data_ptr(), ws.numel(), None)
    assert rc == -1
    rc = L.ffn_swiglu_forward(dX.data_ptr(), dW.data_ptr(), dW.data_ptr(), dWd.data_ptr(),
                              Y.data_ptr(), 4, 64, 256, 64, ffn.BF16, ffn.VARIANT_FUSED,
                              ws.data_ptr(), 0, None)
    assert rc == -2
    torch.cuda.synchronize()
    assert bool((Y.float() == 7.0).all())


def test_swiglu_decode_workload():
    c = workload.SWIGLU_DECODE
    log(f"case {c.name}")
    got, ref, outs = _run(c.M, c.N, c.O, c.P, repeat=2)
    compare(got, ref, BF16_TOL, c.name)
    import torch
    assert torch.equal(outs[0], outs[1]), "two calls differ"


def test_swiglu_prefill_workload():
    c = workload.SWIGLU_PREFILL
    log(f"case {c.name}, every row")
    got, ref, outs = _run(c.M, c.N, c.O, c.P, repeat=2)
    compare(got, ref, BF16_TOL, c.name)
    import torch
    assert torch.equal(outs[0], outs[1]), "two calls differ"
