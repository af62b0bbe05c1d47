"""GPU parity of the MoE layer with the router on the GPU (logits = X Wr + br, the
gate network read as one linear layer), through the C ABI, against the fp64 oracle.

The GPU accumulates the logits in fp32, so a token whose top-k is decided by a
margin below the fp32 rounding of its logits may legitimately route differently
from fp64 logits.  The checks are therefore:
  * every GPU logit lies within the a-priori fp32 summation bound of the fp64
    logit: |l_gpu - l| <= (N + 2) 2^-24 (sum_n |x_n w_n| + |br_e|);
  * the routing integers are bit-exact against the oracle's routing of the GPU's
    own logits (both sides decide from the same fp32 values);
  * every token whose fp64 top-k margin exceeds twice that bound gets the same
    experts as the oracle's routing of the fp64 logits;
  * Y matches the oracle's MoE layer on the GPU's logits within the bf16 rule
    max |Y - Yref| <= 2e-2 rms(Yref), on every token.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import transformer_ffn_fusion_amd as ffn
from transformer_ffn_fusion_amd import synth

from gpu_util import BF16_TOL, compare, dev_bf16, dev_f32, host_f64, log

pytestmark = pytest.mark.gpu


def _logit_bound(X, Wr, br):
    x = np.abs(synth.bf16_bits_to_f32(X).astype(np.float64))
    w = np.abs(synth.bf16_bits_to_f32(Wr).astype(np.float64))
    N = X.shape[1]
    return (N + 2) * 2.0 ** -24 * (x @ w + np.abs(br.astype(np.float64)))


def _check_router(X, Wr, br, k, lg_gpu, ids, w, offs, srt):
    M, E = lg_gpu.shape
    ref = oracle.router_logits(X, Wr, br)
    bound = _logit_bound(X, Wr, br)
    err = np.abs(lg_gpu.astype(np.float64) - ref)
    log(f"  logits: max|err| {err.max():.3e}, max bound {bound.max():.3e}")
    assert np.all(err <= bound), "a GPU logit is outside the fp32 summation bound"
    r_ids, r_w, _, r_offs, r_srt = oracle.moe_route(lg_gpu, k=k)
    assert np.array_equal(ids, r_ids), "top-k ids differ from the routing of the GPU logits"
    assert np.array_equal(offs, r_offs), "expert offsets differ"
    assert np.array_equal(srt, r_srt), "sorted entry lists differ"
    np.testing.assert_allclose(w.astype(np.float64), r_w, rtol=1e-6, atol=1e-7)
    # tokens decided by a clear margin route as the fp64 logits do
    f_ids = oracle.moe_route(ref.astype(np.float32), k=k)[0]
    srt_ref = -np.sort(-ref, axis=1)
    margin = srt_ref[:, k - 1] - (srt_ref[:, k] if k < E else -np.inf)
    clear = margin > 2 * bound.max(axis=1)
    log(f"  {int(clear.sum())} of {M} tokens decided by a clear margin")
    assert np.array_equal(np.sort(ids[clear], axis=1), np.sort(f_ids[clear], axis=1))


@pytest.mark.parametrize("M,E,k,N", [
    (1000, 8, 2, 512),
    (4096, 8, 2, 4096),
    (333, 16, 4, 264),
    (257, 64, 8, 136),
    (17, 256, 1, 64),
])
def test_router_parity(M, E, k, N):
    import torch
    log(f"case router M={M} E={E} k={k} N={N}")
    X, Wr, br, *_ = synth.moe_router_inputs(M, E, N, 8, 8, seed=M + E)
    lg = torch.empty((M, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(M * k, dtype=torch.int32, device="cuda")
    ffn.moe_router(dev_bf16(X), dev_bf16(Wr), dev_f32(br), k, lg, ids, w, offs, srt)
    torch.cuda.synchronize()
    _check_router(X, Wr, br, k, lg.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(),
                  offs.cpu().numpy(), srt.cpu().numpy())


@pytest.mark.parametrize("M,E,k,N,O,P", [
    (130, 8, 2, 128, 512, 264),
    (300, 16, 3, 256, 256, 136),
    (4096, 8, 2, 4096, 2048, 4096),
])
def test_moe_with_router(M, E, k, N, O, P):
    import torch
    log(f"case moe with router M={M} E={E} k={k} N={N} O={O} P={P}")
    X, Wr, br, W1, b1, W2, b2 = synth.moe_router_inputs(M, E, N, O, P, seed=M)
    lg = torch.empty((M, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(M * k, dtype=torch.int32, device="cuda")
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    ffn.moe_ffn_forward_router(dev_bf16(X), dev_bf16(Wr), dev_f32(br), k, dev_bf16(W1), dev_bf16(b1),
                               dev_bf16(W2), dev_bf16(b2), Y, logits_out=lg, topk_ids=ids,
                               topk_w=w, expert_offsets=offs, sorted_entries=srt)
    torch.cuda.synchronize()
    lg_h = lg.cpu().numpy()
    _check_router(X, Wr, br, k, lg_h, ids.cpu().numpy(), w.cpu().numpy(), offs.cpu().numpy(),
                  srt.cpu().numpy())
    ref = oracle.moe_ffn(X, lg_h, W1, b1, W2, b2, k=k)
    compare(host_f64(Y), ref, BF16_TOL, "moe with router")
