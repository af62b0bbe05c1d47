"""GPU parity of the FFN backward (act2 none) through the C ABI against the fp64 oracle.

Every gradient tensor is checked with the bf16 rule of the forward (max |err| <=
2e-2 rms of the reference tensor) plus one bf16 rounding per element
(compare_with_bf16_rounding): the intermediates h, act1'(a) and dY W2^T * act1'(a)
are rounded to bf16 once and enter every product as a factor, the sums accumulate
in fp32; with one token, dW1 is an outer product whose every element keeps the
relative rounding of its da factor (up to 2^-8).  At full size the oracle
computes sampled rows of dX and sampled hidden columns of dW1, db1 and dW2 (rows of
dX and columns of the weight gradients are independent of each other)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import transformer_ffn_fusion_amd as ffn
from transformer_ffn_fusion_amd import synth, workload

from gpu_util import BF16_TOL, compare_with_bf16_rounding, dev_bf16, host_f64, log

pytestmark = pytest.mark.gpu
ACT = {"relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH, "none": oracle.ACT_NONE}


def _run(M, N, O, P, act="gelu_tanh", seed=0, bias=True, rows=None, cols=None, repeat=1):
    import torch
    X, W1, b1, W2, _ = synth.dense_inputs(M, N, O, P, seed=seed, with_bias=bias)
    dY = synth.f32_to_bf16_bits(np.random.default_rng(seed + 1).standard_normal((M, P)).astype(np.float32))
    dX = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dW1 = torch.empty((N, O), dtype=torch.float32, device="cuda")
    db1 = torch.empty(O, dtype=torch.float32, device="cuda")
    dW2 = torch.empty((O, P), dtype=torch.float32, device="cuda")
    db2 = torch.empty(P, dtype=torch.float32, device="cuda")
    ws = ffn.workspace(ffn.ffn_backward_workspace_size(M, N, O, P))
    outs = []
    for _ in range(repeat):
        ffn.ffn_backward(dev_bf16(X), dev_bf16(W1), dev_bf16(b1) if b1 is not None else None,
                         dev_bf16(W2), dev_bf16(dY), dX, dW1, db1, dW2, db2, act1=act, ws=ws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (dX, dW1, db1, dW2, db2)])
    ref = oracle.ffn_backward(X, W1, b1, W2, dY, act1=ACT[act], rows=rows, cols=cols)
    r = slice(None) if rows is None else torch.as_tensor(rows, device="cuda")
    c = slice(None) if cols is None else torch.as_tensor(cols, device="cuda")
    got = (host_f64(dX[r]), host_f64(dW1[:, c]), host_f64(db1[c]), host_f64(dW2[c]), host_f64(db2))
    return got, ref, outs


def _compare_all(got, ref, what):
    for name, g, f in zip(["dX", "dW1", "db1", "dW2", "db2"], got, ref):
        compare_with_bf16_rounding(g, f, BF16_TOL, f"{what} {name}")


@pytest.mark.parametrize("shape", [
    (64, 64, 448, 64),
    (130, 264, 456, 136),    # ragged tiles everywhere, K = M ragged for the weight gradients
    (1, 64, 128, 64),        # one token
    (200, 128, 1024, 512),
])
@pytest.mark.parametrize("act", ["gelu_tanh", "relu", "none"])
def test_backward_shapes(shape, act):
    M, N, O, P = shape
    log(f"case backward {shape} {act}")
    got, ref, _ = _run(M, N, O, P, act=act, seed=M + O)
    _compare_all(got, ref, f"{shape} {act}")


def test_backward_no_bias_and_repeat_bitwise():
    import torch
    log("case backward no bias, two calls")
    got, ref, outs = _run(96, 128, 256, 192, bias=False, repeat=2)
    _compare_all(got, ref, "no bias")
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b), "two calls differ"


def test_backward_prefill_shape_sampled():
    c = workload.PREFILL
    rows = synth.check_rows(c.M, n_random=57)
    cols = np.array([0, 1, 63, 64, 447, 448, 895, 1024, 1790, 1791], dtype=np.int64)
    log(f"case backward {c.name}: {rows.size} rows of dX, {cols.size} hidden columns")
    got, ref, _ = _run(c.M, c.N, c.O, c.P, rows=rows, cols=cols)
    _compare_all(got, ref, c.name)


def test_backward_rejections():
    import torch
    L = ffn.lib()
    z = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    p = z.data_ptr()
    ws = ffn.workspace(ffn.ffn_backward_workspace_size(64, 64, 64, 64))
    # fp32 data: unsupported; unknown activation; workspace too small; misaligned pointer
    assert L.ffn_backward(p, p, None, p, p, p, p, None, p, None, 64, 64, 64, 64, ffn.F32, 2,
                          ws.data_ptr(), ws.numel(), None) == -3
    assert L.ffn_backward(p, p, None, p, p, p, p, None, p, None, 64, 64, 64, 64, ffn.BF16, 7,
                          ws.data_ptr(), ws.numel(), None) == -1
    assert L.ffn_backward(p, p, None, p, p, p, p, None, p, None, 64, 64, 64, 64, ffn.BF16, 2,
                          ws.data_ptr(), 16, None) == -2
    assert L.ffn_backward(p + 8, p, None, p, p, p, p, None, p, None, 64, 64, 64, 64, ffn.BF16, 2,
                          ws.data_ptr(), ws.numel(), None) == -4
    torch.cuda.synchronize()
