"""The C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call
(so these run without a GPU: no call here reaches a kernel launch)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import transformer_ffn_fusion_amd as ffn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffn.h")

E_INVAL, E_WS, E_UNSUP, E_ALIGN = -1, -2, -3, -4
FAKE = 0x10000      # 256-byte aligned, never dereferenced: every call below fails a check first
FAKE2 = 0x20000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text,
                                 flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    L = ffn.lib()
    names = declared_functions()
    assert {"ffn_forward", "ffn_forward_ex", "ffn_workspace_size", "moe_ffn_forward",
            "moe_route", "moe_workspace_size", "ffn_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libffn.so does not export {n}"
    assert L.ffn_version() >= 100


def test_layout_selfcheck():
    assert ffn.lib().ffn_selftest_layout() == 0


def _fwd(X=FAKE, W1=FAKE, b1=None, W2=FAKE, b2=None, Y=FAKE2, M=64, N=64, O=448, P=64,
         dtype=ffn.BF16, act1=2, act2=0, variant=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = 0  # too small unless a test says otherwise
    return ffn.lib().ffn_forward_ex(X, W1, b1, W2, b2, Y, M, N, O, P, dtype, act1, act2, variant,
                                    ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), E_INVAL),
    (dict(M=1 << 20, N=1 << 15, O=1 << 15, P=64), E_UNSUP),
    (dict(N=1 << 24, O=8, P=8), E_UNSUP),    # a 64-row X tile past 32-bit offsets
    (dict(M=16, N=8, O=1 << 24, P=8), E_UNSUP),   # 16 rows of H past 32-bit offsets
    (dict(M=64, N=8, O=8, P=1 << 23), E_UNSUP),   # a 64-row tile of partials past 32-bit offsets
    (dict(W1=None), E_INVAL),
    (dict(Y=None), E_INVAL),
    (dict(ws=None), E_INVAL),
    (dict(M=-1), E_INVAL),
    (dict(N=0), E_INVAL),
    (dict(O=12), E_UNSUP),
    (dict(P=100), E_UNSUP),
    (dict(dtype=7), E_INVAL),
    (dict(act1=5), E_INVAL),
    (dict(act2=-1), E_INVAL),
    (dict(variant=9), E_INVAL),
    (dict(X=FAKE + 8), E_ALIGN),
    (dict(b1=FAKE + 4), E_ALIGN),
    (dict(ws=FAKE + 16), E_ALIGN),
    (dict(variant=ffn.VARIANT_SKINNY, M=17), E_UNSUP),
    (dict(variant=ffn.VARIANT_F32), E_UNSUP),
    (dict(dtype=ffn.F32, variant=ffn.VARIANT_FUSED), E_UNSUP),
    (dict(variant=ffn.VARIANT_DECODE, M=16), E_UNSUP),                    # N, P not 4096
    (dict(variant=ffn.VARIANT_DECODE, M=17, N=4096, O=1792, P=4096), E_UNSUP),
    (dict(variant=ffn.VARIANT_DECODE, M=16, N=4096, O=1920, P=4096), E_UNSUP),  # O % 256
    (dict(variant=ffn.VARIANT_DECODE, M=16, N=4096, O=2304, P=4096), E_UNSUP),  # O > 2048
    (dict(variant=ffn.VARIANT_DECODE, M=16, N=4096, O=1792, P=8192), E_UNSUP),
    (dict(variant=ffn.VARIANT_DECODE, dtype=ffn.F32, M=16, N=4096, O=1792, P=4096), E_UNSUP),
    (dict(), E_WS),
])
def test_forward_rejects(kw, code):
    rc = _fwd(**kw)
    assert rc == code, (rc, ffn.ffn_last_error())
    assert ffn.ffn_last_error() != ""


def test_workspace_one_byte_short_is_rejected():
    need = ffn.ffn_workspace_size(4096, 4096, 1792, 4096)
    assert need >= 4 * 4096 * 4096 * 3          # four packed (3-byte) split partials of Y
    assert _fwd(M=4096, N=4096, O=1792, P=4096, wsb=need - 1) == E_WS
    skinny = ffn.ffn_workspace_size(16, 4096, 1792, 4096)
    assert 0 < skinny < need
    assert _fwd(M=16, N=4096, O=1792, P=4096, wsb=skinny - 1) == E_WS


def test_decode_stream_workspace_sizes():
    # [8][16][16][O/8] fp32 K-block partials, 16 x O bf16 H, [8][16][P] fp32 slice
    # partials, 2 x 256 flags and a status word, each region 256-byte aligned
    dec = ffn.ffn_workspace_size(16, 4096, 1792, 4096, ffn.BF16, ffn.VARIANT_DECODE)
    assert dec == 128 * 16 * 224 * 4 + 16 * 1792 * 2 + 8 * 16 * 4096 * 4 + 2 * 256 * 8 + 256
    skinny_only = ffn.ffn_workspace_size(16, 4096, 1792, 4096, ffn.BF16, ffn.VARIANT_SKINNY)
    auto = ffn.ffn_workspace_size(16, 4096, 1792, 4096)
    assert auto == max(dec, skinny_only)          # AUTO may take either path
    assert _fwd(M=16, N=4096, O=1792, P=4096, variant=ffn.VARIANT_DECODE, wsb=dec - 1) == E_WS
    assert ffn.ffn_workspace_size(16, 4096, 1920, 4096, ffn.BF16, ffn.VARIANT_DECODE) == 0
    assert ffn.ffn_workspace_size(16, 4096, 1792, 4096, ffn.F32, ffn.VARIANT_DECODE) == 0
    # shapes the decode stream does not take keep the skinny size under AUTO
    assert ffn.ffn_workspace_size(16, 4096, 1920, 4096) == \
        ffn.ffn_workspace_size(16, 4096, 1920, 4096, ffn.BF16, ffn.VARIANT_SKINNY)


def test_workspace_size_invalid_shapes():
    assert ffn.ffn_workspace_size(4, 4, 448, 64) == 0
    assert ffn.ffn_workspace_size(4, 64, 448, 64, dtype=5) == 0
    assert ffn.moe_workspace_size(64, 300, 2, 64, 448, 64) == 0
    assert ffn.moe_workspace_size(64, 8, 9, 64, 448, 64) == 0
    assert ffn.moe_workspace_size(64, 2, 3, 64, 448, 64) == 0


def _swiglu(X=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, Y=FAKE2, M=64, N=64, O=256, P=64, dtype=ffn.BF16,
            variant=0, ws=FAKE, wsb=0):
    return ffn.lib().ffn_swiglu_forward(X, Wg, Wu, Wd, Y, M, N, O, P, dtype, variant, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), E_INVAL),
    (dict(Wg=None), E_INVAL),
    (dict(Wu=None), E_INVAL),
    (dict(Wd=None), E_INVAL),
    (dict(Y=None), E_INVAL),
    (dict(ws=None), E_INVAL),
    (dict(M=-1), E_INVAL),
    (dict(O=12), E_UNSUP),
    (dict(dtype=3), E_INVAL),
    (dict(variant=9), E_INVAL),
    (dict(Wu=FAKE + 8), E_ALIGN),
    (dict(Wd=FAKE + 4), E_ALIGN),
    (dict(variant=ffn.VARIANT_SKINNY, M=17), E_UNSUP),
    (dict(dtype=ffn.F32, variant=ffn.VARIANT_SKINNY), E_UNSUP),
    (dict(variant=ffn.VARIANT_DECODE, M=16, N=4096, O=1920, P=4096), E_UNSUP),
    (dict(variant=ffn.VARIANT_DECODE, M=16, N=2048, O=1792, P=4096), E_UNSUP),
    (dict(variant=ffn.VARIANT_DECODE, M=16, N=4096, O=1792, P=4096), E_WS),
    (dict(), E_WS),
])
def test_swiglu_rejects(kw, code):
    rc = _swiglu(**kw)
    assert rc == code, (rc, ffn.ffn_last_error())
    assert ffn.ffn_last_error() != ""


def test_swiglu_workspace_sizes():
    S = ffn.ffn_swiglu_workspace_size
    fused = S(4096, 4096, 1792, 4096)
    assert fused >= 4 * 4096 * 4096 * 3         # four 448-column hidden chunks of packed partials
    assert _swiglu(M=4096, N=4096, O=1792, P=4096, wsb=fused - 1) == E_WS
    dec = S(16, 4096, 1792, 4096)
    assert 0 < dec < fused
    assert _swiglu(M=16, N=4096, O=1792, P=4096, wsb=dec - 1) == E_WS
    assert S(16, 4096, 1792, 4096, ffn.BF16, ffn.VARIANT_FUSED) == 4 * 16 * 4096 * 3
    assert S(16, 4096, 2048, 4096, ffn.BF16, ffn.VARIANT_FUSED) == 8 * 16 * 4096 * 3  # 256-wide
    assert S(4, 4, 448, 64) == 0
    assert S(4, 64, 448, 64, 5) == 0


def _moe(**kw):
    a = dict(X=FAKE, logits=FAKE, M=64, E=8, k=2, W1=FAKE, b1=None, W2=FAKE, b2=None, Y=FAKE2,
             N=64, O=448, P=64, dtype=ffn.BF16, act1=2, act2=0, ws=FAKE, wsb=0)
    a.update(kw)
    return ffn.lib().moe_ffn_forward(a["X"], a["logits"], a["M"], a["E"], a["k"], a["W1"], a["b1"],
                                     a["W2"], a["b2"], a["Y"], a["N"], a["O"], a["P"], a["dtype"],
                                     a["act1"], a["act2"], None, None, None, None, a["ws"],
                                     a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(E=0), E_UNSUP),
    (dict(E=257), E_UNSUP),
    (dict(k=0), E_UNSUP),
    (dict(k=3, E=2), E_UNSUP),
    (dict(k=9, E=16), E_UNSUP),
    (dict(logits=None), E_INVAL),
    (dict(logits=FAKE + 2), E_ALIGN),
    (dict(dtype=ffn.F32), E_UNSUP),
    (dict(O=20), E_UNSUP),
    (dict(act1=3), E_INVAL),
    (dict(W2=FAKE + 4), E_ALIGN),
    (dict(), E_WS),
])
def test_moe_rejects(kw, code):
    rc = _moe(**kw)
    assert rc == code, (rc, ffn.ffn_last_error())


def test_router_rejects():
    L = ffn.lib()
    ws = 1 << 24
    # X, Wr, br, M, N, E, k, logits_out, ids, w, offsets, sorted, ws, bytes, stream
    assert L.moe_router(FAKE, None, None, 64, 64, 8, 2, None, None, None, None, None, FAKE, ws, None) == E_INVAL
    assert L.moe_router(FAKE, FAKE, None, 64, 64, 12, 2, None, None, None, None, None, FAKE, ws, None) == E_UNSUP
    assert L.moe_router(FAKE, FAKE + 8, None, 64, 64, 8, 2, None, None, None, None, None, FAKE, ws, None) == E_ALIGN
    assert L.moe_router(FAKE, FAKE, FAKE + 2, 64, 64, 8, 2, None, None, None, None, None, FAKE, ws, None) == E_ALIGN
    assert L.moe_router(FAKE, FAKE, None, 64, 60, 8, 2, None, None, None, None, None, FAKE, ws, None) == E_UNSUP
    assert L.moe_router(FAKE, FAKE, None, 64, 64, 8, 9, None, None, None, None, None, FAKE, ws, None) == E_UNSUP
    assert L.moe_router(FAKE, FAKE, None, 64, 64, 8, 2, None, None, None, None, None, FAKE, 16, None) == E_WS
    # the full layer: logits come from the router; no Wr is an error
    rc = L.moe_ffn_forward_router(FAKE, None, None, 64, 8, 2, FAKE, None, FAKE, None, FAKE2, 64, 448,
                                  64, ffn.BF16, 2, 0, None, None, None, None, None, FAKE, ws, None)
    assert rc == E_INVAL
    rc = L.moe_ffn_forward_router(FAKE, FAKE, None, 64, 8, 2, FAKE, None, FAKE, None, FAKE2, 64, 448,
                                  64, ffn.BF16, 2, 0, None, None, None, None, None, FAKE, 16, None)
    assert rc == E_WS


def test_backward_rejects_on_host():
    L = ffn.lib()
    args = lambda **kw: dict(dict(X=FAKE, W1=FAKE, b1=None, W2=FAKE, dY=FAKE, dX=FAKE2, dW1=FAKE2,  # noqa: E731
                                  db1=None, dW2=FAKE2, db2=None, M=64, N=64, O=64, P=64,
                                  dt=ffn.BF16, act=2, ws=FAKE, wsb=0), **kw)
    def call(**kw):
        a = args(**kw)
        return L.ffn_backward(a["X"], a["W1"], a["b1"], a["W2"], a["dY"], a["dX"], a["dW1"],
                              a["db1"], a["dW2"], a["db2"], a["M"], a["N"], a["O"], a["P"],
                              a["dt"], a["act"], a["ws"], a["wsb"], None)
    assert call(dt=ffn.F32) == E_UNSUP
    assert call(act=9) == E_INVAL
    assert call(dW1=None) == E_INVAL
    assert call(O=12) == E_UNSUP
    assert call(dY=FAKE + 4) == E_ALIGN
    assert call(M=1 << 20, N=1 << 12) == E_UNSUP
    assert call() == E_WS
    need = ffn.ffn_backward_workspace_size(4096, 4096, 1792, 4096)
    assert need >= 3 * 4096 * 1792 * 2
    assert call(M=4096, N=4096, O=1792, P=4096, wsb=need - 1) == E_WS


def test_route_rejects():
    L = ffn.lib()
    assert L.moe_route(None, 8, 8, 2, None, None, None, None, FAKE, 1 << 20, None) == E_INVAL
    assert L.moe_route(FAKE, 8, 8, 2, None, None, None, None, FAKE, 0, None) == E_WS
    assert L.moe_route(FAKE, 8, 8, 2, None, None, None, None, FAKE + 8, 1 << 20, None) == E_ALIGN


def test_ceiling_entry_points_reject_before_launch():
    """The measurement kernels check their arguments on the host (no GPU needed)."""
    import ctypes
    L = ffn.lib()
    sink_bytes = L.ffn_ceiling_sink_bytes()
    assert L.ffn_ceiling_read(FAKE, 1 << 20, None, sink_bytes, None) == E_INVAL
    assert sink_bytes > 0
    f = ctypes.c_double()
    assert L.ffn_ceiling_mfma(None, sink_bytes, 16, ctypes.byref(f), None) == E_INVAL
    assert L.ffn_ceiling_mfma(FAKE, sink_bytes - 4, 16, ctypes.byref(f), None) == E_WS
    assert L.ffn_ceiling_mfma(FAKE, sink_bytes, 0, ctypes.byref(f), None) == E_INVAL
    assert L.ffn_ceiling_read(FAKE + 4, 1 << 20, FAKE, sink_bytes, None) == E_ALIGN
    assert L.ffn_ceiling_read(FAKE, 24, FAKE, sink_bytes, None) == E_INVAL
    assert L.ffn_ceiling_read(FAKE, 1 << 20, FAKE, 8, None) == E_WS


def test_workspace_follows_the_split_count():
    """The dense fused form's workspace holds the packed (3-byte) partials of its splits:
    448-wide chunks at the prefill shard (4 splits), 896-wide two-pass chunks at
    the large shard (4 splits instead of 8), from the shape alone (no device)."""
    pre = ffn.ffn_workspace_size(4096, 4096, 1792, 4096)
    assert 4 * 4096 * 4096 * 3 <= pre < 5 * 4096 * 4096 * 3
    big = ffn.ffn_workspace_size(8192, 8192, 3584, 8192)
    assert 4 * 8192 * 8192 * 3 <= big < 5 * 8192 * 8192 * 3
    # the GPU parity case of the two-pass form (4090 rows, 7168 hidden): 8 splits, not 16
    two = ffn.ffn_workspace_size(4090, 136, 7168, 1032)
    assert 8 * 4090 * 1032 * 3 <= two < 9 * 4090 * 1032 * 3


def test_noalloc_refuses_shapes_beyond_its_scratch_on_the_host():
    """The size check of ffn_forward_noalloc runs before any HIP call (no GPU here)."""
    L = ffn.lib()
    M, N, O, P = 4096, 4096, 1792, 4096     # 192 MiB of split partials
    assert ffn.ffn_workspace_size(M, N, O, P) > ffn.NOALLOC_SCRATCH_BYTES
    rc = L.ffn_forward_noalloc(FAKE, FAKE, None, FAKE, None, FAKE2, M, N, O, P, ffn.BF16, 2, 0, 0,
                               None)
    assert rc == E_WS, (rc, ffn.ffn_last_error())
    assert "static scratch" in ffn.ffn_last_error()


def test_noalloc_scratch_size_matches_the_header_and_its_stated_shapes():
    text = open(HEADER).read()
    m = re.search(r"#define FFN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << 20\)", text)
    assert m and int(m.group(1)) << 20 == ffn.NOALLOC_SCRATCH_BYTES
    ws = ffn.ffn_workspace_size
    assert ws(16, 4096, 1792, 4096) <= ffn.NOALLOC_SCRATCH_BYTES      # the decode shard
    assert ws(16, 8192, 3584, 8192) <= ffn.NOALLOC_SCRATCH_BYTES      # stated in the header
    assert ws(341, 4096, 1792, 4096) <= ffn.NOALLOC_SCRATCH_BYTES     # stated in the header
    assert ws(342, 4096, 1792, 4096) > ffn.NOALLOC_SCRATCH_BYTES


def test_forward_family_resolution():
    fam = ffn.ffn_forward_family
    assert fam(4096, 4096, 1792, 4096) == ffn.VARIANT_FUSED
    assert fam(8, 128, 512, 128, ffn.F32) == ffn.VARIANT_F32
    assert fam(16, 1024, 896, 1024) == ffn.VARIANT_SKINNY          # not a decode-stream shape
    # the decode stream when the device has 256 CUs (a device count query that fails reads as 256)
    assert fam(16, 4096, 1792, 4096) in (ffn.VARIANT_DECODE, ffn.VARIANT_SKINNY)
    assert fam(16, 4096, 1792, 4096, ffn.BF16, ffn.VARIANT_SKINNY) == ffn.VARIANT_SKINNY
    assert fam(16, 4096, 1792, 4096, ffn.BF16, ffn.VARIANT_DECODE) == ffn.VARIANT_DECODE
    with pytest.raises(ffn.FFNError):
        fam(16, 4096, 1792, 4096, ffn.BF16, 9)
    with pytest.raises(ffn.FFNError):
        fam(16, 4096, 12, 4096)


def test_gated_decode_stream_workspace_sizes():
    S = ffn.ffn_swiglu_workspace_size
    dec = S(16, 4096, 1792, 4096, ffn.BF16, ffn.VARIANT_DECODE)
    # gate and up K-block partials, H, slice partials, flags, status
    assert dec == 2 * 128 * 16 * 224 * 4 + 16 * 1792 * 2 + 8 * 16 * 4096 * 4 + 2 * 256 * 8 + 256
    assert S(16, 4096, 1792, 4096) == max(dec, S(16, 4096, 1792, 4096, ffn.BF16, ffn.VARIANT_SKINNY))
    assert S(16, 4096, 1920, 4096, ffn.BF16, ffn.VARIANT_DECODE) == 0
    assert _swiglu(M=16, N=4096, O=1792, P=4096, variant=ffn.VARIANT_DECODE, wsb=dec - 1) == E_WS


def test_decode_expiry_selftest_checks_its_arguments():
    L = ffn.lib()
    # not a decode-stream shape: refused on the host before any launch
    rc = L.ffn_selftest_decode_expiry(FAKE, FAKE, None, FAKE, None, FAKE2, 16, 1024, 896, 1024, 2, 0,
                                      FAKE, 1 << 30, None)
    assert rc == E_UNSUP, (rc, ffn.ffn_last_error())
    rc = L.ffn_selftest_decode_expiry(FAKE, FAKE, None, FAKE, None, FAKE2, 16, 4096, 1792, 4096, 2, 0,
                                      FAKE, 0, None)
    assert rc == E_WS, (rc, ffn.ffn_last_error())
