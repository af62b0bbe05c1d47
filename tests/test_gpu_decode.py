"""GPU parity of the decode-stream variant (FFN_VARIANT_DECODE): one kernel that
streams W1 and W2 together and passes each XCD's slice of H through that XCD's
L2, then a reduction of the 8 slice partials of Y.

Checked against the fp64 oracle on every row with the plain rule
max |Y - Yref| <= 2e-2 rms(Yref); the flags that order the workgroups carry a
per-call number, so the tests also run calls back to back on one workspace,
alternate input sets, start from a workspace full of random bytes and
interleave the other decode variant on the same workspace.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import transformer_ffn_fusion_amd as ffn
from transformer_ffn_fusion_amd import synth, workload

from gpu_util import BF16_TOL, compare, dev_bf16, host_f64, log

pytestmark = pytest.mark.gpu

ACT = {"relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH, "none": oracle.ACT_NONE}


def _inputs(M, N, O, P, seed, bias=True, bias_var=0.02):
    return synth.dense_inputs(M, N, O, P, seed=seed, with_bias=bias, bias_var=bias_var)


def _dev(arrs):
    return [dev_bf16(a) if a is not None else None for a in arrs]


def _call(dev, Y, ws, variant=ffn.VARIANT_DECODE, act1="gelu_tanh", act2="none"):
    X, W1, b1, W2, b2 = dev
    ffn.ffn_forward_ex(X, W1, b1, W2, b2, Y, act1, act2, variant, ws)


def _ref(host, act1="gelu_tanh", act2="none"):
    X, W1, b1, W2, b2 = host
    return oracle.ffn(X, W1, b1, W2, b2, act1=ACT[act1], act2=ACT[act2])


@pytest.mark.parametrize("shape", [
    (16, 4096, 1792, 4096),   # the decode shard
    (1, 4096, 1792, 4096),    # one token
    (5, 4096, 256, 4096),     # one 32-column step per XCD
    (11, 4096, 2048, 4096),   # the widest slice (256 columns per XCD)
    (16, 4096, 768, 4096),    # 96 columns per XCD: a partly filled column block
])
def test_decode_stream_shapes(shape):
    import torch
    M, N, O, P = shape
    log(f"case decode stream {shape}")
    host = _inputs(M, N, O, P, seed=M * 13 + O)
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    ws = ffn.workspace(ffn.ffn_workspace_size(M, N, O, P, ffn.BF16, ffn.VARIANT_DECODE))
    _call(_dev(host), Y, ws)
    torch.cuda.synchronize()
    compare(host_f64(Y), _ref(host), BF16_TOL, f"decode stream {shape}")


@pytest.mark.parametrize("act1,act2,bias", [("relu", "none", True), ("none", "gelu_tanh", True),
                                            ("gelu_tanh", "relu", False)])
def test_decode_stream_activations_and_bias(act1, act2, bias):
    import torch
    M, N, O, P = 7, 4096, 1024, 4096
    log(f"case decode stream act {act1}/{act2} bias {bias}")
    host = _inputs(M, N, O, P, seed=5, bias=bias, bias_var=0.5)
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    ws = ffn.workspace(ffn.ffn_workspace_size(M, N, O, P, ffn.BF16, ffn.VARIANT_DECODE))
    _call(_dev(host), Y, ws, act1=act1, act2=act2)
    torch.cuda.synchronize()
    compare(host_f64(Y), _ref(host, act1, act2), BF16_TOL, f"act {act1}/{act2}")


def test_decode_stream_calls_in_a_row_on_one_workspace():
    """Alternating input sets on one workspace that starts as random bytes, with
    the four-kernel decode variant run on the same workspace in between: every
    call matches its own reference, and repeated calls give the same bits."""
    import torch
    c = workload.DECODE
    log(f"case decode stream, calls in a row ({c.name})")
    hosts = [_inputs(c.M, c.N, c.O, c.P, seed=s) for s in (31, 32)]
    devs = [_dev(h) for h in hosts]
    refs = [_ref(h) for h in hosts]
    nbytes = ffn.ffn_workspace_size(c.M, c.N, c.O, c.P, ffn.BF16)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda",
                       generator=torch.Generator(device="cuda").manual_seed(33))
    first = [None, None]
    for i in range(6):
        s = i % 2
        Y = torch.empty((c.M, c.P), dtype=torch.bfloat16, device="cuda")
        _call(devs[s], Y, ws)
        if i == 3:   # the other variant overwrites the shared regions
            Ys = torch.empty_like(Y)
            _call(devs[1 - s], Ys, ws, variant=ffn.VARIANT_SKINNY)
            torch.cuda.synchronize()
            compare(host_f64(Ys), refs[1 - s], BF16_TOL, "skinny in between")
        torch.cuda.synchronize()
        if first[s] is None:
            compare(host_f64(Y), refs[s], BF16_TOL, f"call {i} (set {s})")
            first[s] = Y
        else:
            assert torch.equal(Y, first[s]), f"call {i}: set {s} gave other bits"


def test_decode_stream_is_the_default_and_matches_skinny():
    import torch
    c = workload.DECODE
    log(f"case decode stream vs skinny ({c.name})")
    host = _inputs(c.M, c.N, c.O, c.P, seed=41)
    dev = _dev(host)
    ref = _ref(host)
    outs = {}
    for v in (ffn.VARIANT_AUTO, ffn.VARIANT_DECODE, ffn.VARIANT_SKINNY):
        Y = torch.empty((c.M, c.P), dtype=torch.bfloat16, device="cuda")
        ws = ffn.workspace(ffn.ffn_workspace_size(c.M, c.N, c.O, c.P, ffn.BF16, v))
        _call(dev, Y, ws, variant=v)
        torch.cuda.synchronize()
        compare(host_f64(Y), ref, BF16_TOL, f"variant {v}")
        outs[v] = Y
    assert torch.equal(outs[ffn.VARIANT_AUTO], outs[ffn.VARIANT_DECODE])


# ---------------------------------------------------------------- gated (SwiGLU) form

def _swiglu(M, N, O, P, seed, variant, ws=None, repeat=1):
    import torch
    X, Wg, Wu, Wd = synth.swiglu_inputs(M, N, O, P, seed=seed)
    dev = [dev_bf16(a) for a in (X, Wg, Wu, Wd)]
    if ws is None:
        ws = ffn.workspace(ffn.ffn_swiglu_workspace_size(M, N, O, P, ffn.BF16, variant))
    outs = []
    for _ in range(repeat):
        Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
        ffn.ffn_swiglu_forward(*dev, Y, variant, ws)
        torch.cuda.synchronize()
        outs.append(Y)
    return outs, oracle.swiglu(X, Wg, Wu, Wd)


@pytest.mark.parametrize("shape", [
    (16, 4096, 1792, 4096),   # the SwiGLU decode shard
    (3, 4096, 512, 4096),
    (9, 4096, 2048, 4096),
])
def test_gated_decode_stream_shapes(shape):
    M, N, O, P = shape
    log(f"case gated decode stream {shape}")
    outs, ref = _swiglu(M, N, O, P, seed=M + O, variant=ffn.VARIANT_DECODE, repeat=2)
    compare(host_f64(outs[0]), ref, BF16_TOL, f"gated decode stream {shape}")
    import torch
    assert torch.equal(outs[0], outs[1]), "two calls differ"


def test_gated_decode_stream_is_the_default_and_matches_skinny():
    import torch
    c = workload.SWIGLU_DECODE
    log(f"case gated decode stream vs skinny ({c.name})")
    got = {}
    for v in (ffn.VARIANT_AUTO, ffn.VARIANT_DECODE, ffn.VARIANT_SKINNY):
        outs, ref = _swiglu(c.M, c.N, c.O, c.P, seed=51, variant=v)
        compare(host_f64(outs[0]), ref, BF16_TOL, f"variant {v}")
        got[v] = outs[0]
    assert torch.equal(got[ffn.VARIANT_AUTO], got[ffn.VARIANT_DECODE])


def test_decode_stream_expired_wait_poisons_output():
    """The failure path, forced from the host: the self-test entry point runs the
    call with flags that never match and waits of 64 polls, so every wait
    expires; Y must be NaN everywhere, and the next call on the same workspace
    must be right again."""
    import torch
    c = workload.DECODE
    log(f"case decode stream, expired waits ({c.name})")
    host = _inputs(c.M, c.N, c.O, c.P, seed=61)
    X, W1, b1, W2, b2 = _dev(host)
    Y = torch.zeros((c.M, c.P), dtype=torch.bfloat16, device="cuda")
    ws = ffn.workspace(ffn.ffn_workspace_size(c.M, c.N, c.O, c.P, ffn.BF16, ffn.VARIANT_DECODE))
    stream = torch.cuda.current_stream().cuda_stream
    rc = ffn.lib().ffn_selftest_decode_expiry(X.data_ptr(), W1.data_ptr(), b1.data_ptr(),
                                              W2.data_ptr(), b2.data_ptr(), Y.data_ptr(), c.M, c.N,
                                              c.O, c.P, ffn.ACT_GELU_TANH, ffn.ACT_NONE,
                                              ws.data_ptr(), ws.numel(), stream)
    assert rc == 0, ffn.ffn_last_error()
    torch.cuda.synchronize()
    assert bool(torch.isnan(Y.float()).all()), "an expired wait must poison every element"
    Y2 = torch.empty_like(Y)
    _call([X, W1, b1, W2, b2], Y2, ws)
    torch.cuda.synchronize()
    compare(host_f64(Y2), _ref(host), BF16_TOL, "the call after the expired one")
