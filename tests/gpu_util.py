"""Helpers for the GPU parity tests: moving the seeded inputs to the device and
comparing the library's outputs with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

BF16_TOL = 2e-2   # max |Y - Yref| <= BF16_TOL * rms(Yref): bf16 data, fp32 accumulation
F32_TOL = 1e-5    # same rule for fp32 data


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def compare(y_gpu, y_ref, tol, what=""):
    """Max-abs error against tol * rms of the reference; returns (max_err, rms)."""
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    log(f"  {what}: max|err| = {err:.3e}, rms(ref) = {rms:.3e}, ratio = {err / max(rms, 1e-30):.3e}"
        f" (tol {tol:.0e})")
    assert err <= tol * rms, f"{what}: max|err| {err:.4e} > {tol} * rms {rms:.4e}"
    return err, rms


def compare_with_bf16_rounding(y_gpu, y_ref, tol, what=""):
    """As ``compare``, with one bf16 rounding per element added to the allowance:
    |Y - Yref| <= tol * rms(Yref) + 2^-8 |Yref|.

    bf16 keeps 8 significant bits, so rounding to nearest moves a value y by at most
    half an ulp, 2^-8 |y| (reached just above a power of two; 2^-9 |y| is only the
    typical size).  For a gradient whose terms are products with one bf16-rounded
    factor (da or h), a short sum (one token: an outer product) keeps that factor's
    relative rounding error on every element, and the largest elements of a product
    of two normal draws are ~12 rms.  2^-8 |Yref| covers one such rounding.  The
    forward outputs are checked with ``compare`` (the plain rule) instead."""
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = np.abs(y_gpu - y_ref)
    excess = float(np.max(err - 2.0 ** -8 * np.abs(y_ref))) if y_ref.size else 0.0
    log(f"  {what}: max|err| = {float(err.max()) if err.size else 0.0:.3e} "
        f"({(float(err.max()) if err.size else 0.0) / max(rms, 1e-30):.3e} rms); "
        f"beyond one bf16 rounding: {excess / max(rms, 1e-30):.3e} rms (tol {tol:.0e})")
    assert excess <= tol * rms, f"{what}: error beyond one bf16 rounding {excess:.4e} > {tol} * rms {rms:.4e}"
