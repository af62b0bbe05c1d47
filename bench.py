#!/usr/bin/env python3
"""Benchmark of the fused FFN on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload prefill|decode|large|moe|tiny|swiglu|swiglu_decode] [--all]

A step is one call of the whole path on one batch of synthetic input that is
already resident in HBM: for the dense workloads the fused FFN kernel and the
ordered split reduction (at M <= 16: the decode streaming kernel and its slice
reduction, or the two skinny layers where the streaming kernel does not apply); for the MoE
workload routing, the grouped fused FFN and the combine; for the backward
workload the six steps of the gradients at the prefill shape; for the SwiGLU
workloads the gated fused FFN and the reduction (two gated skinny layers at
M <= 16).  W untimed warm-up
steps, then K timed steps bracketed by a device synchronisation on both sides
(region 1, the headline value), then K more steps with HIP events recorded on
the launch stream before, between and after the kernels (region 2, the
per-kernel durations behind `roofline`; an event mark costs a few
microseconds of gap, so region 1 carries none).

Inputs are rotated over R identical copies (R * bytes >= 512 MB) so that the
256 MB Infinity Cache cannot serve the weights from one call to the next.  The
dense workloads then run K more plain steps on one input set (region 3, no
rotation): `warm_ms_per_step`, a warm-cache figure reported beside the
headline, never as it; then, once the process has made SETTLE_CALLS calls
(untimed ones make up the difference), K more rotated steps (region 4):
`settled`, the rate after the GPU's start-up ramp (from an idle GPU the first
~140 calls of a process run up to ~40 % slower; after the box-ceiling kernels'
~120 ms of load, calls 6-25 still run ~7 % slower than settled), also beside
the headline, never as it.

One JSON line goes to stdout:
  value      whole-path throughput of the headline workload (TFLOP/s at M=4096);
  roofline   the dominant kernel's algorithmic FLOPs (or bytes) per launch over its
             average duration, timed live with HIP events recorded on the launch
             stream around each kernel, against MI355X's published peak;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same workload;
  box_ceilings  this GPU's own bf16 MFMA and HBM-read ceilings, measured in the same
             run right before the headline workload's warm-up steps, after ~120 ms
             of back-to-back launches of both kernels, which also take the GPU out
             of its idle power state (roofline carries the fraction of the
             measured ceiling);
  secondary  the decode shape (M=16: us/call, HBM GB/s) and, with --all, the others.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

METRIC = ("fused FFN TFLOP/s and % bf16 MFMA peak at M=4096; "
          "µs/call + HBM GB/s at M=16")
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (AMD published, no sparsity)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
MALL_DEFEAT_BYTES = 512 << 20
SETTLE_CALLS = 300   # calls after which the path runs at its settled rate (region 4)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")
COPY_BYTES = 256 << 20   # the plain copy used to calibrate the HBM byte counters


# the sources of the kernels whose HBM traffic is recorded (forward fused and grouped,
# decode stream and layers, routing and combine, and the headers they include)
TRAFFIC_SOURCES = ("ffn_fused.hip", "ffn_skinny.hip", "ffn_decode.hip", "moe.hip", "ffn_backward.hip",
                   "ffn_device.h", "ffn_internal.h")


def kernel_source_hash() -> str:
    """Hash of the measured kernels' sources: traffic counters are valid only for them."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "transformer_ffn_fusion_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload_name: str):
    """HBM bytes per launch of the dominant kernel, from profiles/traffic.json, or None
    when the record is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload_name)
    return None if w is None else w.get("hbm_bytes_per_launch")


def copy_calibration():
    """One plain device-to-device copy of COPY_BYTES (for counter calibration runs)."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


class Hip:
    """The few HIP runtime calls the bench makes itself (events)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self, device_only=False):
        """A timing event; device_only events skip the system-scope fence (hipEventDisableSystemFence),
        which the per-kernel marks inside a step do not need: they are only compared on the device."""
        e = ctypes.c_void_p()
        if device_only:
            assert self.h.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000) == 0
        else:
            assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.h.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.h.hipEventSynchronize(b) == 0
        assert self.h.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(e)


def to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------------- dense

def run_dense(cfg, steps, warmup, hip, torch, ffn, synth, workload, prelude=None):
    """Dense FFN workloads, and the SwiGLU ones (cfg a workload.Gated: its inputs
    are X, Wg, Wu, Wd and it has no biases)."""
    dt = cfg.dtype
    gated = isinstance(cfg, workload.Gated)
    es = workload.esize(dt)
    if gated:
        X, W1, b1, W2 = synth.swiglu_inputs(cfg.M, cfg.N, cfg.O, cfg.P, dtype=dt, seed=0)
        b2 = None
        set_bytes = workload.swiglu_bytes(cfg.M, cfg.N, cfg.O, cfg.P, es)
    else:
        X, W1, b1, W2, b2 = synth.dense_inputs(cfg.M, cfg.N, cfg.O, cfg.P, dtype=dt,
                                               bias_var=cfg.bias_var, seed=0)
        set_bytes = workload.dense_bytes(cfg.M, cfg.N, cfg.O, cfg.P, es)
    # gated: the slots (X, W1, b1, W2, b2) hold X, Wg, Wu, Wd and no b2
    R = max(1, min(64, math.ceil(MALL_DEFEAT_BYTES / set_bytes)))
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    base = [to_dev(a, torch) for a in (X, W1, b1, W2, b2)]
    sets = [[None if t is None else t.clone() for t in base] + [torch.empty((cfg.M, cfg.P), dtype=tdt, device="cuda")]
            for _ in range(R)]
    del base
    code = ffn.BF16 if dt == "bf16" else ffn.F32
    if gated:
        ws = ffn.workspace(ffn.ffn_swiglu_workspace_size(cfg.M, cfg.N, cfg.O, cfg.P, code))
    else:
        ws = ffn.workspace(ffn.ffn_workspace_size(cfg.M, cfg.N, cfg.O, cfg.P, code))
    L = ffn.lib()
    stream = torch.cuda.current_stream().cuda_stream
    act1 = 0 if gated else ffn.ACTS[cfg.act1]
    nev = 3
    evs = [hip.event(device_only=True) for _ in range(nev * steps)]
    arr_t = ctypes.c_void_p * nev

    def call(i, ev=None):
        x, w1, c1, w2, c2, y = sets[i % R]
        p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        if gated and ev is None:
            rc = L.ffn_swiglu_forward(p(x), p(w1), p(c1), p(w2), p(y), cfg.M, cfg.N, cfg.O, cfg.P,
                                      code, 0, p(ws), ws.numel(), stream)
        elif gated:
            rc = L.ffn_swiglu_forward_traced(p(x), p(w1), p(c1), p(w2), p(y), cfg.M, cfg.N, cfg.O,
                                             cfg.P, code, 0, p(ws), ws.numel(), stream, ev, nev)
        elif ev is None:
            rc = L.ffn_forward(p(x), p(w1), p(c1), p(w2), p(c2), p(y), cfg.M, cfg.N, cfg.O, cfg.P,
                               code, act1, 0, p(ws), ws.numel(), stream)
        else:
            rc = L.ffn_forward_traced(p(x), p(w1), p(c1), p(w2), p(c2), p(y), cfg.M, cfg.N, cfg.O,
                                      cfg.P, code, act1, 0, 0, p(ws), ws.numel(), stream, ev, nev)
        if rc != 0:
            raise RuntimeError(ffn.ffn_last_error())

    if prelude is not None:
        prelude()
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # timed region 1: K plain steps -> the headline value
    t0, t1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hip.record(t0, stream)
    for s in range(steps):
        call(s)
    hip.record(t1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = hip.ms(t0, t1)
    # timed region 2: the same K steps with an event before, between and after
    # the two kernels -> per-kernel durations (the events themselves add a gap
    # at every mark, so they stay out of region 1)
    ev_arrays = [arr_t(*evs[nev * s: nev * (s + 1)]) for s in range(steps)]
    t2, t3 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(t2, stream)
    for s in range(steps):
        call(steps + s, ev_arrays[s])
    hip.record(t3, stream)
    torch.cuda.synchronize()
    traced_ms = hip.ms(t2, t3)
    k1 = [hip.ms(evs[nev * s], evs[nev * s + 1]) for s in range(steps)]
    k2 = [hip.ms(evs[nev * s + 1], evs[nev * s + 2]) for s in range(steps)]
    # timed region 3: the same K plain steps on ONE input set (no rotation), so
    # the inputs can stay in the 256 MB memory-side cache from call to call;
    # reported beside the headline under its own name, never as the headline
    for _ in range(10):
        call(0)
    t4, t5 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(t4, stream)
    for s in range(steps):
        call(0)
    hip.record(t5, stream)
    torch.cuda.synchronize()
    warm_ms = hip.ms(t4, t5)
    # region 4: the same K rotated steps once the GPU has left its start-up
    # ramp (from an idle GPU calls take up to ~40 % longer over the first ~140
    # calls of a process; after the box-ceiling kernels' load, a few per cent):
    # untimed calls up to SETTLE_CALLS in all, then K timed ones ->
    # `settled_ms_per_step`, reported beside the headline, never as it
    done = warmup + 2 * steps + 10 + steps
    for i in range(max(0, SETTLE_CALLS - done)):
        call(i)
    t6, t7 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(t6, stream)
    for s in range(steps):
        call(s)
    hip.record(t7, stream)
    torch.cuda.synchronize()
    settled_ms = hip.ms(t6, t7)
    hip.destroy(evs + [t0, t1, t2, t3, t4, t5, t6, t7])
    flops = (workload.swiglu_flops if gated else workload.dense_flops)(cfg.M, cfg.N, cfg.O, cfg.P)
    nbytes = set_bytes
    ms = total_ms / steps
    return dict(ms_per_step=ms, wall_ms_per_step=1e3 * wall / steps,
                traced_ms_per_step=traced_ms / steps, k1_ms=float(np.mean(k1)),
                k1_std_ms=float(np.std(k1)), k2_ms=float(np.mean(k2)), flops=flops, bytes=nbytes,
                warm_ms_per_step=warm_ms / steps, settled_ms_per_step=settled_ms / steps,
                settled_after_calls=max(done, SETTLE_CALLS), rotate=R,
                # the SwiGLU form resolves its family by the same rule as the dense one
                family=ffn.ffn_forward_family(cfg.M, cfg.N, cfg.O, cfg.P, code),
                inputs=(X, W1, b1, W2, b2))


def run_moe_router(cfg, steps, warmup, hip, torch, ffn, synth, workload, prelude=None):
    """The MoE layer with the router on the GPU (logits = X Wr + br): region 1 times
    the whole layer, region 2 the router + routing alone."""
    X, Wr, br, W1, b1, W2, b2 = synth.moe_router_inputs(cfg.M, cfg.E, cfg.N, cfg.O, cfg.P, seed=0)
    set_bytes = workload.moe_bytes(cfg.M, cfg.E, cfg.N, cfg.O, cfg.P) + 2 * cfg.N * cfg.E
    R = max(1, min(8, math.ceil(MALL_DEFEAT_BYTES / set_bytes)))
    base = [to_dev(a, torch) for a in (X, Wr, br, W1, b1, W2, b2)]
    sets = [[t.clone() for t in base] +
            [torch.empty((cfg.M, cfg.P), dtype=torch.bfloat16, device="cuda")] for _ in range(R)]
    del base
    ws = ffn.workspace(ffn.moe_workspace_size(cfg.M, cfg.E, cfg.k, cfg.N, cfg.O, cfg.P))
    L = ffn.lib()
    stream = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()  # noqa: E731

    def layer(i):
        x, wr, c, w1, c1, w2, c2, y = sets[i % R]
        rc = L.moe_ffn_forward_router(p(x), p(wr), p(c), cfg.M, cfg.E, cfg.k, p(w1), p(c1), p(w2),
                                      p(c2), p(y), cfg.N, cfg.O, cfg.P, ffn.BF16, 2, 0, None, None,
                                      None, None, None, p(ws), ws.numel(), stream)
        if rc != 0:
            raise RuntimeError(ffn.ffn_last_error())

    def route(i):
        x, wr, c = sets[i % R][:3]
        rc = L.moe_router(p(x), p(wr), p(c), cfg.M, cfg.N, cfg.E, cfg.k, None, None, None, None,
                          None, p(ws), ws.numel(), stream)
        if rc != 0:
            raise RuntimeError(ffn.ffn_last_error())

    if prelude is not None:
        prelude()
    for i in range(warmup):
        layer(i)
    torch.cuda.synchronize()
    t0, t1, t2, t3 = hip.event(), hip.event(), hip.event(), hip.event()
    hip.record(t0, stream)
    for s_ in range(steps):
        layer(s_)
    hip.record(t1, stream)
    torch.cuda.synchronize()
    hip.record(t2, stream)
    for s_ in range(steps):
        route(steps + s_)
    hip.record(t3, stream)
    torch.cuda.synchronize()
    total_ms, route_ms = hip.ms(t0, t1), hip.ms(t2, t3)
    hip.destroy([t0, t1, t2, t3])
    flops = workload.moe_flops(cfg.M * cfg.k, cfg.N, cfg.O, cfg.P) + 2 * cfg.M * cfg.N * cfg.E
    return dict(ms_per_step=total_ms / steps, router_ms=route_ms / steps, flops=flops,
                bytes=set_bytes, rotate=R)


def run_moe(cfg, steps, warmup, hip, torch, ffn, synth, workload, prelude=None):
    # the workload's gate logits are X Wr + offsets: formed once, before any
    # timing, by the library's router (then an input of every timed call)
    X, Wr, br, W1, b1, W2, b2 = synth.moe_router_inputs(cfg.M, cfg.E, cfg.N, cfg.O, cfg.P, seed=0)
    logits = torch.empty((cfg.M, cfg.E), dtype=torch.float32, device="cuda")
    ffn.moe_router(to_dev(X, torch), to_dev(Wr, torch), to_dev(br, torch), cfg.k, logits_out=logits)
    torch.cuda.synchronize()
    set_bytes = workload.moe_bytes(cfg.M, cfg.E, cfg.N, cfg.O, cfg.P)
    R = max(1, min(8, math.ceil(MALL_DEFEAT_BYTES / set_bytes)))
    base = [to_dev(X, torch), logits] + [to_dev(a, torch) for a in (W1, b1, W2, b2)]
    sets = [[t.clone() for t in base] +
            [torch.empty((cfg.M, cfg.P), dtype=torch.bfloat16, device="cuda")] for _ in range(R)]
    del base
    ws = ffn.workspace(ffn.moe_workspace_size(cfg.M, cfg.E, cfg.k, cfg.N, cfg.O, cfg.P))
    L = ffn.lib()
    stream = torch.cuda.current_stream().cuda_stream
    nev = 4
    evs = [hip.event(device_only=True) for _ in range(nev * steps)]
    arr_t = ctypes.c_void_p * nev

    def call(i, ev=None):
        x, lg, w1, c1, w2, c2, y = sets[i % R]
        p = lambda t: t.data_ptr()  # noqa: E731
        if ev is None:
            rc = L.moe_ffn_forward(p(x), p(lg), cfg.M, cfg.E, cfg.k, p(w1), p(c1), p(w2), p(c2),
                                   p(y), cfg.N, cfg.O, cfg.P, ffn.BF16, 2, 0, None, None, None,
                                   None, p(ws), ws.numel(), stream)
        else:
            rc = L.moe_ffn_forward_traced(p(x), p(lg), cfg.M, cfg.E, cfg.k, p(w1), p(c1), p(w2),
                                          p(c2), p(y), cfg.N, cfg.O, cfg.P, ffn.BF16, 2, 0,
                                          p(ws), ws.numel(), stream, ev, nev)
        if rc != 0:
            raise RuntimeError(ffn.ffn_last_error())

    if prelude is not None:
        prelude()
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, stream)
    for s in range(steps):          # timed region 1: plain steps
        call(s)
    hip.record(t1, stream)
    torch.cuda.synchronize()
    total_ms = hip.ms(t0, t1)
    ev_arrays = [arr_t(*evs[nev * s: nev * (s + 1)]) for s in range(steps)]
    t2, t3 = hip.event(), hip.event()
    hip.record(t2, stream)
    for s in range(steps):          # timed region 2: the same steps, marked per kernel
        call(steps + s, ev_arrays[s])
    hip.record(t3, stream)
    torch.cuda.synchronize()
    traced_ms = hip.ms(t2, t3)
    ks = [[hip.ms(evs[nev * s + j], evs[nev * s + j + 1]) for s in range(steps)] for j in range(3)]
    hip.destroy(evs + [t0, t1, t2, t3])
    flops = workload.moe_flops(cfg.M * cfg.k, cfg.N, cfg.O, cfg.P)
    return dict(ms_per_step=total_ms / steps, traced_ms_per_step=traced_ms / steps,
                route_ms=float(np.mean(ks[0])),
                k1_ms=float(np.mean(ks[1])), combine_ms=float(np.mean(ks[2])), flops=flops,
                bytes=set_bytes, rotate=R)


def run_backward(cfg, steps, warmup, hip, torch, ffn, synth, workload, prelude=None):
    """The FFN backward at a dense shape (act2 none): region 1 plain calls, region 2
    the same calls with events between the six steps."""
    X, W1, b1, W2, _ = synth.dense_inputs(cfg.M, cfg.N, cfg.O, cfg.P, seed=0)
    dY = synth.f32_to_bf16_bits(np.random.default_rng(1).standard_normal((cfg.M, cfg.P)).astype(np.float32))
    set_bytes = 2 * (cfg.M * cfg.N + cfg.N * cfg.O + cfg.O + cfg.O * cfg.P + cfg.M * cfg.P)
    R = max(1, min(16, math.ceil(MALL_DEFEAT_BYTES / set_bytes)))
    base = [to_dev(a, torch) for a in (X, W1, b1, W2, dY)]
    sets = [[t.clone() for t in base] for _ in range(R)]
    del base
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")  # noqa: E731
    dX = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device="cuda")
    dW1, db1, dW2, db2 = f32(cfg.N, cfg.O), f32(cfg.O), f32(cfg.O, cfg.P), f32(cfg.P)
    ws = ffn.workspace(ffn.ffn_backward_workspace_size(cfg.M, cfg.N, cfg.O, cfg.P))
    L = ffn.lib()
    stream = torch.cuda.current_stream().cuda_stream
    act = ffn.ACTS[cfg.act1]
    nev = 7
    evs = [hip.event(device_only=True) for _ in range(nev * steps)]
    arr_t = ctypes.c_void_p * nev
    p = lambda t: t.data_ptr()  # noqa: E731

    def call(i, ev=None):
        x, w1, c1, w2, dy = sets[i % R]
        a = (p(x), p(w1), p(c1), p(w2), p(dy), p(dX), p(dW1), p(db1), p(dW2), p(db2), cfg.M, cfg.N,
             cfg.O, cfg.P, ffn.BF16, act, p(ws), ws.numel(), stream)
        rc = L.ffn_backward(*a) if ev is None else L.ffn_backward_traced(*a, ev, nev)
        if rc != 0:
            raise RuntimeError(ffn.ffn_last_error())

    if prelude is not None:
        prelude()
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, stream)
    for s_ in range(steps):
        call(s_)
    hip.record(t1, stream)
    torch.cuda.synchronize()
    total_ms = hip.ms(t0, t1)
    ev_arrays = [arr_t(*evs[nev * s_: nev * (s_ + 1)]) for s_ in range(steps)]
    for s_ in range(steps):
        call(steps + s_, ev_arrays[s_])
    torch.cuda.synchronize()
    names = ["h_and_grad", "da", "dX", "dW1", "dW2", "bias_sums"]
    per = {n: float(np.mean([hip.ms(evs[nev * s_ + j], evs[nev * s_ + j + 1]) for s_ in range(steps)]))
           for j, n in enumerate(names)}
    hip.destroy(evs + [t0, t1])
    gemm = 2 * cfg.M * cfg.N * cfg.O   # each of the five products: 2 M N O = 2 M O P here
    flops_alg = 2 * cfg.M * (2 * cfg.N * cfg.O + 2 * cfg.O * cfg.P)   # dh, dX, dW1, dW2
    flops_exec = flops_alg + gemm                                        # + the recomputed a
    return dict(ms_per_step=total_ms / steps, steps_ms=per, flops=flops_alg, flops_exec=flops_exec,
                bytes=set_bytes, rotate=R)


# ---------------------------------------------------------------- box ceilings

def box_ceilings(hip, torch, ffn, reps=10, busy_ms=120.0):
    """This GPU's own ceilings, measured in the same run: a loop of independent
    bf16 MFMAs on register operands, and a streaming read of a 1 GiB buffer
    (four times the Infinity Cache).

    It runs right before the headline workload's warm-up steps: both kernels are
    first launched back to back for `busy_ms`, then timed.  From idle, the GPU
    needs some ~100 ms of continuous load to leave its low-power state (measured
    on MI355X: prefill calls 11-60 of a fresh process took 200-222 us each from
    idle, 181-192 us after 100 ms of these kernels, and a 1 s idle gap after
    them undid it), so the ceilings are timed on a busy GPU and the workload
    that follows starts from the same state whatever its warm-up count."""
    L = ffn.lib()
    sink = torch.zeros(L.ffn_ceiling_sink_bytes() // 4, dtype=torch.float32, device="cuda")
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    t_busy = time.perf_counter()
    while (time.perf_counter() - t_busy) * 1e3 < busy_ms:
        for _ in range(4):
            ffn.ceiling_mfma(sink, 2048)
            ffn.ceiling_read(buf, sink)
        torch.cuda.synchronize()
    busy = (time.perf_counter() - t_busy) * 1e3
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, stream)
    for _ in range(reps):
        flops = ffn.ceiling_mfma(sink, 2048)
    hip.record(t1, stream)
    mfma_ms = hip.ms(t0, t1) / reps
    hip.record(t0, stream)
    for _ in range(reps):
        nbytes = ffn.ceiling_read(buf, sink)
    hip.record(t1, stream)
    read_ms = hip.ms(t0, t1) / reps
    hip.destroy([t0, t1])
    del buf
    return {"mfma_bf16_tflops": flops / (mfma_ms * 1e-3) / 1e12,
            "hbm_read_gbs": nbytes / (read_ms * 1e-3) / 1e9,
            "how": "loop of independent v_mfma_f32_16x16x32_bf16 (2048 workgroups x 4 waves); "
                   "16-byte streaming read of 1 GiB; both launched back to back for %.0f ms, then "
                   "the mean of %d launches each; run right before the headline workload's "
                   "warm-up steps" % (busy, reps)}


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(cfg, inputs, rows, synth, workload):
    import oracle  # the reported CPU baseline is the oracle as it stands
    X, W1, b1, W2, b2 = inputs
    sel = np.arange(rows, dtype=np.int64)
    gated = isinstance(cfg, workload.Gated)
    t0 = time.perf_counter()
    if gated:
        oracle.swiglu(X, W1, b1, W2, rows=sel)
    else:
        oracle.ffn(X, W1, b1, W2, b2, act1=oracle.ACT_GELU_TANH, rows=sel)
    dt = time.perf_counter() - t0
    flops = (workload.swiglu_flops if gated else workload.dense_flops)(rows, cfg.N, cfg.O, cfg.P)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": (f"the whole call, {rows} rows of {cfg.name} (fp64, {dt:.2f} s)"
                       if rows == cfg.M else
                       f"{rows} of {cfg.M} rows of {cfg.name} (fp64, {dt:.2f} s); "
                       f"extrapolated full call {dt * cfg.M / rows:.1f} s")}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # untimed steps first: the first ~20 ms of back-to-back calls run up to
    # 10 % slower (221 -> 199 us per prefill call over the first 300 calls)
    # while the GPU settles, so the timed steps start in the steady state
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "decode", "large", "moe", "tiny", "swiglu", "swiglu_decode",
                             "moe_shard", "backward"])
    ap.add_argument("--all", action="store_true", help="also time the large and MoE workloads")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="oracle rows (default: the whole prefill call, ~1.5 s on 16 host threads; 0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run one plain 256 MiB device copy (to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the path runs on a single MI355X, no cross-GPU step is built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_ffn_fusion_amd as ffn
    from transformer_ffn_fusion_amd import synth, workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ffn.lib()  # fail loudly when the library is missing
    hip = Hip()
    cfgs = {"prefill": workload.PREFILL, "decode": workload.DECODE, "large": workload.LARGE,
            "tiny": workload.TINY_F32, "moe": workload.MOE, "swiglu": workload.SWIGLU_PREFILL,
            "swiglu_decode": workload.SWIGLU_DECODE, "moe_shard": workload.MOE_SHARD,
            "backward": workload.PREFILL}
    head = cfgs[args.workload]
    log(f"[bench] device {torch.cuda.get_device_name(0)}; workload {head.name}")

    ceil = {}

    def prelude():
        ceil.update(box_ceilings(hip, torch, ffn))

    secondary = {}
    if args.workload == "backward":
        r = run_backward(head, args.steps, args.warmup, hip, torch, ffn, synth, workload, prelude)
        r["traced_ms_per_step"] = sum(r["steps_ms"].values())
        value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
        unit = "TFLOP/s"
        dom = "h_and_grad"   # the first product (recomputes H and act1'(a)): the longest step
        gemm_flops = 2 * head.M * head.N * head.O
        ach = gemm_flops / (r["steps_ms"][dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": f"backward GEMM ({dom})", "achieved": ach,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                "traffic": recorded_traffic(head.name), "kernel_us": 1e3 * r["steps_ms"][dom],
                "steps_us": {k: 1e3 * v for k, v in r["steps_ms"].items()},
                "executed_TFLOP_per_s": r["flops_exec"] / (r["ms_per_step"] * 1e-3) / 1e12}
        dense = None
    elif args.workload in ("moe", "moe_shard"):
        r = run_moe(head, args.steps, args.warmup, hip, torch, ffn, synth, workload, prelude)
        value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
        kern_tflops = r["flops"] / (r["k1_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "grouped fused FFN", "achieved": kern_tflops,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": kern_tflops / PEAK_BF16_TFLOPS,
                "traffic": recorded_traffic(head.name), "kernel_us": 1e3 * r["k1_ms"],
                "route_us": 1e3 * r["route_ms"], "combine_us": 1e3 * r["combine_ms"]}
        unit = "TFLOP/s"
        dense = None
    else:
        r = run_dense(head, args.steps, args.warmup, hip, torch, ffn, synth, workload, prelude)
        dense = r
        if head.M <= 16 and head.dtype == "bf16":
            value = r["bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
            unit = "GB/s"
            if r["family"] == ffn.VARIANT_DECODE and isinstance(head, workload.Gated):
                # the gated streaming kernel reads X, Wg, Wu and Wd and writes the 8
                # slice partials of Y (16 rows x P fp32 each)
                k1_bytes = (2 * (head.M * head.N + 2 * head.N * head.O + head.O * head.P)
                            + 8 * 16 * head.P * 4)
                kname = "gated decode streaming kernel (both layers, H through each XCD's L2)"
            elif r["family"] == ffn.VARIANT_DECODE:
                # the streaming kernel reads X, W1, b1 and W2 and writes the 8 slice
                # partials of Y (16 rows x P fp32 each); the slice reduction follows
                k1_bytes = (2 * (head.M * head.N + head.N * head.O + head.O + head.O * head.P)
                            + 8 * 16 * head.P * 4)
                kname = "decode streaming kernel (both layers, H through each XCD's L2)"
            elif isinstance(head, workload.Gated):
                # skinny layers: layer 1 streams Wg and Wu (no bias) and writes H
                k1_bytes = 2 * (head.M * head.N + 2 * head.N * head.O + head.M * head.O)
                kname = "gated skinny layer 1 (stream + ordered reduce)"
            else:
                k1_bytes = 2 * (head.M * head.N + head.N * head.O + head.O + head.M * head.O)
                kname = "skinny layer 1 (stream + ordered reduce)"
            ach = k1_bytes / (r["k1_ms"] * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": kname, "achieved": ach,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                    "traffic": recorded_traffic(head.name), "kernel_us": 1e3 * r["k1_ms"],
                    "second_kernel_us": 1e3 * r["k2_ms"]}
        else:
            value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
            unit = "TFLOP/s"
            ach = r["flops"] / (r["k1_ms"] * 1e-3) / 1e12
            peak = PEAK_BF16_TFLOPS if head.dtype == "bf16" else 157.3
            kname = "gated fused FFN (H in LDS)" if isinstance(head, workload.Gated) else "fused FFN (H in LDS)"
            roof = {"bound": "mfma", "kernel": kname, "achieved": ach, "peak": peak,
                    "unit": "TFLOP/s", "frac": ach / peak, "traffic": recorded_traffic(head.name),
                    "kernel_us": 1e3 * r["k1_ms"], "reduce_us": 1e3 * r["k2_ms"]}

    if args.workload == "prefill":
        d = run_dense(workload.DECODE, max(args.steps, 200), args.warmup, hip, torch, ffn, synth,
                      workload)
        secondary[workload.DECODE.name] = {
            "us_per_call": 1e3 * d["ms_per_step"],
            "GB_per_s": d["bytes"] / (d["ms_per_step"] * 1e-3) / 1e9,
            "frac_hbm_peak": d["bytes"] / (d["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "path": "decode stream" if d["family"] == ffn.VARIANT_DECODE else "skinny layers",
            "kernel1_us": 1e3 * d["k1_ms"], "kernel2_us": 1e3 * d["k2_ms"],
            "kernels_GB_per_s": d["bytes"] / ((d["k1_ms"] + d["k2_ms"]) * 1e-3) / 1e9,
            "rotate": d["rotate"], "warm_us_per_call": 1e3 * d["warm_ms_per_step"],
            "settled_us_per_call": 1e3 * d["settled_ms_per_step"]}
    if args.all:
        for name in ("large", "moe", "moe_shard", "tiny", "swiglu", "swiglu_decode"):
            c = cfgs[name]
            if c is head:
                continue
            if name in ("moe", "moe_shard"):
                m = run_moe(c, args.steps, args.warmup, hip, torch, ffn, synth, workload)
                secondary[c.name] = {"TFLOP_per_s": m["flops"] / (m["ms_per_step"] * 1e-3) / 1e12,
                                     "us_per_call": 1e3 * m["ms_per_step"],
                                     "route_us": 1e3 * m["route_ms"],
                                     "grouped_us": 1e3 * m["k1_ms"],
                                     "combine_us": 1e3 * m["combine_ms"]}
            else:
                m = run_dense(c, args.steps, args.warmup, hip, torch, ffn, synth, workload)
                secondary[c.name] = {"TFLOP_per_s": m["flops"] / (m["ms_per_step"] * 1e-3) / 1e12,
                                     "GB_per_s": m["bytes"] / (m["ms_per_step"] * 1e-3) / 1e9,
                                     "us_per_call": 1e3 * m["ms_per_step"],
                                     "kernel1_us": 1e3 * m["k1_ms"], "kernel2_us": 1e3 * m["k2_ms"]}

    if args.all:
        b = run_backward(workload.PREFILL, args.steps, args.warmup, hip, torch, ffn, synth, workload)
        secondary["backward_" + workload.PREFILL.name] = {
            "TFLOP_per_s": b["flops"] / (b["ms_per_step"] * 1e-3) / 1e12,
            "us_per_call": 1e3 * b["ms_per_step"],
            "steps_us": {k: round(1e3 * v, 1) for k, v in b["steps_ms"].items()}}
        m = run_moe_router(workload.MOE, args.steps, args.warmup, hip, torch, ffn, synth, workload)
        secondary["moe_router_" + workload.MOE.name] = {
            "TFLOP_per_s": m["flops"] / (m["ms_per_step"] * 1e-3) / 1e12,
            "us_per_call": 1e3 * m["ms_per_step"], "router_and_routing_us": 1e3 * m["router_ms"]}

    if roof["unit"] == "TFLOP/s" and head.dtype == "bf16":
        roof["measured_peak"] = ceil["mfma_bf16_tflops"]
        roof["frac_of_measured_peak"] = roof["achieved"] / ceil["mfma_bf16_tflops"]
    elif roof["unit"] == "GB/s":
        roof["measured_peak"] = ceil["hbm_read_gbs"]
        roof["frac_of_measured_peak"] = roof["achieved"] / ceil["hbm_read_gbs"]

    cpu = None
    if dense is not None and args.cpu_rows > 0 and head.dtype == "bf16":
        rows = min(args.cpu_rows, head.M)
        log(f"[bench] CPU oracle baseline on {rows} rows ...")
        cpu = cpu_baseline(head, dense["inputs"], rows, synth, workload)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "traced_ms_per_step": r["traced_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.dtype,
        "data": "synthetic (seeded normal inputs, random-init weights of the workload's shape)",
        "config": {"workload": ("backward_" if args.workload == "backward" else "") + head.name,
                   **{k: getattr(head, k) for k in ("M", "N", "O", "P")},
                   "act1": getattr(head, "act1", "swiglu"), "rotate_input_sets": r["rotate"]},
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS if unit == "TFLOP/s" else None,
        "roofline": roof,
        "cpu_baseline": cpu,
        "warm_ms_per_step": r.get("warm_ms_per_step"),
        "settled": None if r.get("settled_ms_per_step") is None else {
            "ms_per_step": r["settled_ms_per_step"], "after_calls": r["settled_after_calls"],
            "value": (value * r["ms_per_step"] / r["settled_ms_per_step"]) if unit == "TFLOP/s" else None},
        "box_ceilings": ceil,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
