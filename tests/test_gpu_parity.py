"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case uses the seeded generators of ``transformer_ffn_fusion_amd.synth``
for both sides.  Tolerance: max |Y - Yref| <= 2e-2 * rms(Yref) for bf16 data
with fp32 accumulation, <= 1e-5 * rms(Yref) for fp32 data, over the checked
elements.  Rows of Y depend only on the same row of X (the FFN equations act
row by row), so a sampled row is an exact check of that row.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import transformer_ffn_fusion_amd as ffn
from transformer_ffn_fusion_amd import synth, workload

from gpu_util import (BF16_TOL, F32_TOL, compare, compare_with_bf16_rounding, dev_bf16, dev_f32,
                      host_f64, log)

pytestmark = pytest.mark.gpu

ACT = {"relu": oracle.ACT_RELU, "gelu_tanh": oracle.ACT_GELU_TANH, "none": oracle.ACT_NONE}


def _run_dense(M, N, O, P, *, dtype="bf16", act1="gelu_tanh", act2="none", variant=0,
               seed=0, bias=True, bias_var=0.02, rows=None, repeat=1):
    import torch
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, dtype=dtype, seed=seed, with_bias=bias,
                                           bias_var=bias_var)
    to = dev_bf16 if dtype == "bf16" else dev_f32
    dX, dW1, dW2 = to(X), to(W1), to(W2)
    db1 = to(b1) if b1 is not None else None
    db2 = to(b2) if b2 is not None else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Y = torch.empty((M, P), dtype=tdt, device="cuda")
    ws = ffn.workspace(ffn.ffn_workspace_size(M, N, O, P, ffn.BF16 if dtype == "bf16" else ffn.F32,
                                              variant))
    outs = []
    for _ in range(repeat):
        ffn.ffn_forward_ex(dX, dW1, db1, dW2, db2, Y, act1, act2, variant, ws)
        torch.cuda.synchronize()
        outs.append(Y.clone())
    ref = oracle.ffn(X, W1, b1, W2, b2, act1=ACT[act1], act2=ACT[act2], rows=rows)
    got = host_f64(Y if rows is None else Y[torch.as_tensor(rows, device="cuda")])
    return got, ref, outs


# ---------------------------------------------------------------- shapes and tails

@pytest.mark.parametrize("shape", [
    (1, 64, 448, 512),       # one row, one chunk, one output pass
    (65, 264, 456, 520),     # ragged rows, k tail, ragged chunk, ragged output pass
    (130, 512, 1792, 1032),  # 4 chunks of 448, 3 row tiles (last ragged)
    (200, 128, 1024, 64),    # chunk 512 x2, narrow output
    (64, 1000, 904, 1544),   # ragged everywhere, 2 chunks of 512 (second ragged)
])
def test_fused_shapes(shape):
    M, N, O, P = shape
    log(f"case fused {shape}")
    got, ref, _ = _run_dense(M, N, O, P, variant=ffn.VARIANT_FUSED, seed=M + N)
    compare(got, ref, BF16_TOL, f"fused {shape}")


@pytest.mark.parametrize("shape", [
    (1, 256, 128, 128),
    (5, 520, 264, 136),       # ragged K blocks and column blocks
    (16, 4096, 1792, 4096),
    (16, 1024, 3584, 512),
    (9, 8192, 256, 1024),
    (7, 520, 1000, 2056),     # layer 2 over the whole K: K tail inside a step, ragged last block
    (16, 256, 2048, 2048),    # layer 2 over the whole K in two load batches
])
def test_skinny_shapes(shape):
    M, N, O, P = shape
    log(f"case skinny {shape}")
    got, ref, _ = _run_dense(M, N, O, P, variant=ffn.VARIANT_SKINNY, seed=M * 7 + P)
    compare(got, ref, BF16_TOL, f"skinny {shape}")


def test_fused_and_skinny_agree_at_m16():
    M, N, O, P = 16, 1024, 896, 1024
    log("case fused vs skinny at M=16")
    a, ref, _ = _run_dense(M, N, O, P, variant=ffn.VARIANT_FUSED)
    b, _, _ = _run_dense(M, N, O, P, variant=ffn.VARIANT_SKINNY)
    compare(a, ref, BF16_TOL, "fused M=16")
    compare(b, ref, BF16_TOL, "skinny M=16")


@pytest.mark.parametrize("act1,act2", [("relu", "none"), ("none", "none"), ("gelu_tanh", "relu"),
                                       ("relu", "gelu_tanh")])
@pytest.mark.parametrize("variant", [ffn.VARIANT_FUSED, ffn.VARIANT_SKINNY])
def test_activations(act1, act2, variant):
    M = 70 if variant == ffn.VARIANT_FUSED else 11
    log(f"case act {act1}/{act2} variant {variant}")
    got, ref, _ = _run_dense(M, 256, 512, 264, act1=act1, act2=act2, variant=variant, bias_var=0.5)
    compare(got, ref, BF16_TOL, f"act {act1}/{act2}")


@pytest.mark.parametrize("variant", [ffn.VARIANT_FUSED, ffn.VARIANT_SKINNY])
def test_no_bias(variant):
    M = 33 if variant == ffn.VARIANT_FUSED else 3
    log(f"case no bias variant {variant}")
    got, ref, _ = _run_dense(M, 128, 448, 256, bias=False, variant=variant)
    compare(got, ref, BF16_TOL, "no bias")


@pytest.mark.parametrize("shape", [(3, 40, 520, 72), (130, 136, 1104, 264), (8, 128, 512, 128)])
def test_fp32_shapes(shape):
    M, N, O, P = shape
    log(f"case fp32 {shape}")
    got, ref, _ = _run_dense(M, N, O, P, dtype="f32", act1="relu", bias_var=0.1)
    compare(got, ref, F32_TOL, f"fp32 {shape}")


def test_tensor_parallel_shards():
    """Each shard's partial (b2 on shard 0 only) matches the oracle's partial; the
    sum of the GPU partials matches the unsharded FFN."""
    import torch
    M, N, O, P, G = 96, 512, 1792, 512, 4
    log("case tensor-parallel shards")
    X, W1, b1, W2, b2 = synth.dense_inputs(M, N, O, P, seed=17)
    full = oracle.ffn(X, W1, b1, W2, b2)
    w = O // G
    total = np.zeros((M, P))
    for g in range(G):
        sl = slice(g * w, (g + 1) * w)
        W1g, b1g, W2g = (np.ascontiguousarray(a) for a in (W1[:, sl], b1[sl], W2[sl, :]))
        b2g = b2 if g == 0 else None
        Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
        ffn.ffn_forward(dev_bf16(X), dev_bf16(W1g), dev_bf16(b1g), dev_bf16(W2g),
                        dev_bf16(b2g) if b2g is not None else None, Y)
        torch.cuda.synchronize()
        part = host_f64(Y)
        compare(part, oracle.ffn(X, W1g, b1g, W2g, b2g), BF16_TOL, f"shard {g}")
        total += part
    compare(total, full, BF16_TOL, "sum of shards")


def test_zero_rows_is_noop_and_errors_leave_output_untouched():
    import torch
    M, N, O, P = 4, 64, 448, 64
    X, W1, b1, W2, b2 = (dev_bf16(a) for a in synth.dense_inputs(M, N, O, P))
    Y = torch.full((M, P), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = ffn.workspace(ffn.ffn_workspace_size(M, N, O, P))
    ffn.ffn_forward(X[:0], W1, b1, W2, b2, Y[:0], ws=ws)
    with pytest.raises(ffn.FFNError):
        ffn.ffn_forward(X, W1, b1, W2, b2, Y, ws=ws[:100])
    with pytest.raises(ffn.FFNError):
        ffn.ffn_forward_ex(X, W1, b1, W2, b2, Y, act1=9, ws=ws)
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())


# ---------------------------------------------------------------- MoE

def moe_layer_inputs(M, E, N, O, P, *, seed=0, offsets=synth.MOE_SKEW_OFFSETS):
    """MoE inputs with the gate logits formed as the workload states them: one linear
    router, logits = X Wr + offsets (the MoE review, zhongzhuzhou.org, section 2.2,
    step 1: each token runs the gate).  The oracle sums in fp64 and the result is
    rounded once to fp32; both sides then route from the same fp32 array."""
    X, Wr, br, W1, b1, W2, b2 = synth.moe_router_inputs(M, E, N, O, P, seed=seed, offsets=offsets)
    logits = oracle.router_logits(X, Wr, br).astype(np.float32)
    return X, logits, W1, b1, W2, b2


def _run_moe(M, E, k, N, O, P, *, seed=0, offsets=synth.MOE_SKEW_OFFSETS, rows=None,
             check_all_rows=False, router_logits=False):
    import torch
    if router_logits:
        X, logits, W1, b1, W2, b2 = moe_layer_inputs(M, E, N, O, P, seed=seed, offsets=offsets)
    else:
        X, logits, W1, b1, W2, b2 = synth.moe_inputs(M, E, N, O, P, seed=seed, offsets=offsets)
    dX, dl = dev_bf16(X), dev_f32(logits)
    Y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((M, k), dtype=torch.float32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(M * k, dtype=torch.int32, device="cuda")
    ffn.moe_ffn_forward(dX, dl, k, dev_bf16(W1), dev_bf16(b1), dev_bf16(W2), dev_bf16(b2), Y,
                        topk_ids=ids, topk_w=wts, expert_offsets=offs, sorted_entries=srt)
    torch.cuda.synchronize()
    r_ids, r_w, r_counts, r_offs, r_srt = oracle.moe_route(logits, k=k)
    # integer routing outputs: bit-exact, every token
    assert np.array_equal(ids.cpu().numpy(), r_ids), "top-k ids differ"
    assert np.array_equal(offs.cpu().numpy(), r_offs), "expert offsets differ"
    assert np.array_equal(srt.cpu().numpy(), r_srt), "sorted entry lists differ"
    np.testing.assert_allclose(wts.cpu().numpy().astype(np.float64), r_w, rtol=1e-6, atol=1e-7)
    if rows is None:
        if check_all_rows:
            rows = np.arange(M)
        else:
            rows = set(synth.check_rows(M, n_random=min(249, M)).tolist())
            for e in range(E):   # first and last entry of every expert's list
                seg = r_srt[r_offs[e]:r_offs[e + 1]]
                if seg.size:
                    rows |= {int(seg[0]) // k, int(seg[-1]) // k}
            small = int(np.argmin(r_counts))
            seg = r_srt[r_offs[small]:r_offs[small + 1]]
            rows |= set((seg[:4] // k).tolist())
            rows = np.array(sorted(rows))
    ref = oracle.moe_ffn(X, logits, W1, b1, W2, b2, k=k, rows=rows)
    got = host_f64(Y[torch.as_tensor(rows, device="cuda")])
    return got, ref, r_counts


def test_moe_workload():
    """The MoE workload as configured (router logits X Wr + offsets), every token."""
    c = workload.MOE
    log(f"case {c.name}, every token")
    got, ref, counts = _run_moe(c.M, c.E, c.k, c.N, c.O, c.P, router_logits=True,
                                check_all_rows=True)
    log(f"  expert loads {counts.tolist()}")
    compare(got, ref, BF16_TOL, c.name)


def test_moe_workload_drawn_logits_sampled():
    """The same layer with the logits drawn directly (normal + offset): sampled rows,
    the first and last token of every expert list."""
    c = workload.MOE
    log(f"case {c.name}, drawn logits, sampled tokens")
    got, ref, _ = _run_moe(c.M, c.E, c.k, c.N, c.O, c.P)
    compare(got, ref, BF16_TOL, c.name + " (drawn logits)")


@pytest.mark.parametrize("M,E,k,N,O,P", [
    (50, 4, 1, 64, 448, 128),
    (130, 8, 2, 128, 512, 264),
    (257, 5, 3, 64, 904, 72),
    (64, 1, 1, 256, 448, 512),
    (100, 4, 2, 128, 512, 4096),   # a short round: each unit cut into 8 pass ranges
    (300, 8, 2, 64, 1024, 2048),   # 2 chunks, pass ranges of a 4-pass output
    (200, 64, 2, 64, 448, 128),    # many experts, a few tokens each, some with none
    (90, 256, 1, 64, 256, 64),     # the largest expert count: most experts receive no token
])
def test_moe_shapes(M, E, k, N, O, P):
    log(f"case moe M={M} E={E} k={k} N={N} O={O} P={P}")
    got, ref, _ = _run_moe(M, E, k, N, O, P, seed=M, offsets=(0.5, -0.5, 0.25, 0, 0.1, 0, 0, 0),
                           check_all_rows=True)
    compare(got, ref, BF16_TOL, "moe")


def test_moe_expert_shard_workload():
    """One GPU's share of an 8-way expert-sharded layer: every expert at O = 256, the
    router logits of the full layer, every token."""
    c = workload.MOE_SHARD
    log(f"case {c.name}, every token")
    got, ref, counts = _run_moe(c.M, c.E, c.k, c.N, c.O, c.P, router_logits=True,
                                check_all_rows=True)
    log(f"  expert loads {counts.tolist()}")
    compare(got, ref, BF16_TOL, c.name)


def test_fused_two_pass_chunk_sampled_rows():
    """Where 448-wide chunks would give four or more full rounds of units, each
    workgroup covers 896 hidden columns in two first-product passes (half the
    splits): 64 row tiles (the last ragged) x 8 splits, ragged K and output pass."""
    M, N, O, P = 4090, 136, 7168, 1032
    rows = synth.check_rows(M)
    rows = np.union1d(rows, np.arange(4032, M))   # every row of the ragged last tile
    log(f"case fused two-pass chunk {(M, N, O, P)}, {rows.size} rows")
    got, ref, outs = _run_dense(M, N, O, P, variant=ffn.VARIANT_FUSED, seed=31, rows=rows, repeat=2)
    compare(got, ref, BF16_TOL, "fused two-pass chunk")
    import torch
    assert torch.equal(outs[0], outs[1]), "two calls differ"


def test_fused_partial_plane_past_2GiB():
    """A split's plane of packed partials larger than 2^31 bytes (65536 rows x
    16384 columns x 3 bytes = 3 GiB): the kernel addresses each tile's rows
    through a buffer resource based at the tile, so no offset passes 2^31;
    sampled rows, the last row tile's among them, against the oracle."""
    M, N, O, P = 65536, 64, 448, 16384
    assert M * P * 3 > (1 << 31)
    log(f"case fused, 3 GiB partial plane {(M, N, O, P)}")
    rows = sorted(set(range(0, M, 4099)) | {M - 64, M - 1})
    got, ref, _ = _run_dense(M, N, O, P, variant=ffn.VARIANT_FUSED, seed=77, rows=rows)
    compare(got, ref, BF16_TOL, "3 GiB partial plane")


@pytest.mark.parametrize("shape", [(100, 256, 256, 520), (70, 64, 136, 64)])
def test_fused_narrow_hidden(shape):
    """Hidden widths of at most 256 run the 256-wide chunk."""
    M, N, O, P = shape
    log(f"case fused narrow {shape}")
    got, ref, _ = _run_dense(M, N, O, P, variant=ffn.VARIANT_FUSED, seed=O)
    compare(got, ref, BF16_TOL, f"fused {shape}")


@pytest.mark.parametrize("M,E,k", [
    (1000, 8, 2),
    (3000, 64, 8),    # several staged logit blocks (128 tokens each), k at its maximum
    (700, 256, 5),    # the largest expert count: 32 tokens per staged block
    (1, 3, 3),        # one token, every expert picked
])
def test_moe_route_ties_bit_exact(M, E, k):
    import torch
    log(f"case moe route M={M} E={E} k={k}")
    rng = np.random.default_rng(5 + E)
    logits = (rng.integers(-3, 4, size=(M, E)) * 0.5).astype(np.float32)
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(M * k, dtype=torch.int32, device="cuda")
    ffn.moe_route(dev_f32(logits), k, ids, w, offs, srt)
    torch.cuda.synchronize()
    r_ids, r_w, _, r_offs, r_srt = oracle.moe_route(logits, k=k)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert np.array_equal(offs.cpu().numpy(), r_offs)
    assert np.array_equal(srt.cpu().numpy(), r_srt)
    np.testing.assert_allclose(w.cpu().numpy(), r_w, rtol=1e-6)


# ---------------------------------------------------------------- the five workloads

def test_tiny_fp32_workload():
    c = workload.TINY_F32
    log(f"case {c.name}")
    got, ref, _ = _run_dense(c.M, c.N, c.O, c.P, dtype="f32", act1="relu", bias_var=c.bias_var)
    compare(got, ref, F32_TOL, c.name)


def test_decode_workload():
    c = workload.DECODE
    log(f"case {c.name}")
    got, ref, outs = _run_dense(c.M, c.N, c.O, c.P, repeat=2)
    compare(got, ref, BF16_TOL, c.name)
    import torch
    assert torch.equal(outs[0], outs[1]), "two calls differ"


def test_prefill_workload():
    c = workload.PREFILL
    log(f"case {c.name}, every row")
    got, ref, outs = _run_dense(c.M, c.N, c.O, c.P, repeat=2)
    compare(got, ref, BF16_TOL, c.name)
    import torch
    assert torch.equal(outs[0], outs[1]), "two calls differ"


def test_large_workload():
    c = workload.LARGE
    log(f"case {c.name}, every row")
    got, ref, _ = _run_dense(c.M, c.N, c.O, c.P)
    compare(got, ref, BF16_TOL, c.name)


def test_ceiling_kernels_run():
    """The measurement-support kernels run and report their work (no parity: they compute nothing)."""
    import torch
    sink = torch.zeros(ffn.lib().ffn_ceiling_sink_bytes() // 4, dtype=torch.float32, device="cuda")
    flops = ffn.ceiling_mfma(sink, 4)
    buf = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    nbytes = ffn.ceiling_read(buf, sink)
    torch.cuda.synchronize()
    assert flops == 2048 * 4 * 4 * 8 * (2.0 * 16 * 16 * 32)
    assert nbytes == 1 << 20
    assert float(sink.abs().sum()) == 0.0   # the sink is never written


# ---------------------------------------------------------------- every row at full size
#
# A row of Y depends on its own row of X only (and, for MoE, on its own
# logits).  Permuting the tokens must therefore permute the output rows; this
# checks every row of the full-size workloads without the oracle.  Bitwise
# where the summation order of every output element is fixed by its column
# alone (decode: the K blocks of a column are summed in ascending order
# whatever the row; MoE routing: integers).  The fused and grouped kernels
# start each unit's k-loops at a stage rotated by the unit's index (to spread
# the L2 traffic of units that stream the same weights), so a row's summation
# order depends on the tile it lands in: each call is bitwise reproducible, but
# a permuted call agrees with the original only to the two outputs' bf16
# roundings, |a - b| <= 2e-2 rms + 2^-8 |b|, on every row.


def _rows_agree(got, ref, bitwise, what):
    import torch
    assert bool(torch.isfinite(got.float()).all()), f"{what}: non-finite output"
    if bitwise:
        assert torch.equal(got, ref), f"{what}: permuted rows give different bits"
    else:
        compare_with_bf16_rounding(host_f64(got), host_f64(ref), BF16_TOL, what)


@pytest.mark.parametrize("which", ["prefill", "decode"])
def test_rows_permutation_equivariant(which):
    import torch
    c = workload.PREFILL if which == "prefill" else workload.DECODE
    log(f"case row permutation {c.name}")
    X, W1, b1, W2, b2 = (dev_bf16(a) for a in synth.dense_inputs(c.M, c.N, c.O, c.P, seed=21))
    perm = torch.as_tensor(np.random.default_rng(22).permutation(c.M), device="cuda")
    Y = torch.empty((c.M, c.P), dtype=torch.bfloat16, device="cuda")
    Yp = torch.empty_like(Y)
    ffn.ffn_forward(X, W1, b1, W2, b2, Y)
    ffn.ffn_forward(X[perm].contiguous(), W1, b1, W2, b2, Yp)
    torch.cuda.synchronize()
    _rows_agree(Yp, Y[perm], which == "decode", f"row permutation {c.name}")


def test_moe_tokens_permutation_equivariant():
    import torch
    c = workload.MOE
    log(f"case token permutation {c.name}")
    X, lg, W1, b1, W2, b2 = synth.moe_inputs(c.M, c.E, c.N, c.O, c.P, seed=23)
    dX, dW1, db1, dW2, db2 = (dev_bf16(a) for a in (X, W1, b1, W2, b2))
    dl = dev_f32(lg)
    perm = torch.as_tensor(np.random.default_rng(24).permutation(c.M), device="cuda")
    outs = []
    for xs, ls in ((dX, dl), (dX[perm].contiguous(), dl[perm].contiguous())):
        Y = torch.empty((c.M, c.P), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((c.M, c.k), dtype=torch.int32, device="cuda")
        ffn.moe_ffn_forward(xs, ls, c.k, dW1, db1, dW2, db2, Y, topk_ids=ids)
        outs.append((Y, ids))
    torch.cuda.synchronize()
    (Y, ids), (Yp, idsp) = outs
    assert torch.equal(idsp, ids[perm]), "permuted tokens route differently"
    _rows_agree(Yp, Y[perm], False, f"token permutation {c.name}")
