"""The C-ABI library: it loads, exports every symbol include/dsc.h declares, and
rejects bad arguments with the documented status before enqueuing anything.

Runs without a GPU: every call here fails validation (or is the B*T == 0 no-op),
so no HIP call is made. Pointers are plain integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import dynamic_short_convolutions_amd as dsc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsc.LIB_PATH), reason="libdsc.so not built")

OK, INVALID, MISALIGNED, ALIASING, NOT_SUPPORTED, WORKSPACE, HIPERR = range(7)
F32, BF16 = dsc.DSC_F32, dsc.DSC_BF16
A = 1 << 20  # fake, 16-byte aligned "device addresses", far apart
X, Wp, Y, DY, DX, DW, Z, UU, DZ, DU = (A * (i + 1) * 64 for i in range(10))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsc_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(dsc.EXPORTED)
    L = ctypes.CDLL(dsc.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert dsc.dsc_abi_version() == 8
    for code, name in dsc.STATUS_NAMES.items():
        assert dsc.dsc_status_string(code).startswith(name)
    assert "unknown" in dsc.dsc_status_string(99)


def fwd(x=X, w=Wp, y=Y, B=2, T=8, D=64, G=8, W=4, res=1, dt=BF16):
    return dsc.lib().dsc_fwd(x, w, y, B, T, D, G, W, res, dt, None)


def bwd(x=X, w=Wp, dy=DY, dx=DX, dw=DW, B=2, T=8, D=64, G=8, W=4, res=1, dt=BF16):
    return dsc.lib().dsc_bwd(x, w, dy, dx, dw, B, T, D, G, W, res, dt, None)


def lfwd(x=X, z=Z, U=UU, y=Y, B=2, T=8, D=64, R=16, W=4, res=0, dt=BF16):
    return dsc.lib().dsc_lowrank_fwd(x, z, U, y, B, T, D, R, W, res, dt, None)


WS = A * 1000  # a fake workspace far from the other fake buffers, with room to spare


def lbwd(x=X, z=Z, U=UU, dy=DY, dx=DX, dz=DZ, dU=DU, ws=WS, wsb=1 << 40, B=2, T=8, D=64, R=16, W=4, res=0, dt=BF16):
    return dsc.lib().dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, ws, wsb, B, T, D, R, W, res, dt, None)


@pytest.mark.parametrize("call", [fwd, bwd, lfwd, lbwd])
def test_empty_problem_is_a_noop(call):
    assert call(B=0) == OK
    assert call(T=0) == OK
    assert call(B=0, x=None) == OK          # nothing is read when there is nothing to do


@pytest.mark.parametrize("call", [fwd, bwd, lfwd, lbwd])
def test_invalid_values(call):
    assert call(B=-1) == INVALID
    assert call(T=-3) == INVALID
    assert call(D=0) == INVALID
    assert call(W=0) == INVALID
    assert call(W=9) == INVALID
    assert call(dt=7) == INVALID
    assert call(res=2) == INVALID
    assert call(x=None) == INVALID


def test_head_count_must_divide_channels():
    assert fwd(G=0) == INVALID
    assert fwd(G=5) == INVALID   # 64 % 5 != 0
    assert bwd(G=-8) == INVALID
    # 24 % 3 == 0 passes this check; the aliasing check (the last before a launch) then stops it
    assert fwd(G=3, D=24, y=X) == ALIASING


def test_rank_bounds():
    assert lfwd(R=0) == INVALID
    assert lfwd(R=129) == INVALID
    assert lbwd(R=0) == INVALID


@pytest.mark.parametrize("call,arg", [(fwd, "w"), (fwd, "y"), (bwd, "dx"), (bwd, "dw"), (lfwd, "U"), (lbwd, "dz")])
def test_null_pointers(call, arg):
    assert call(**{arg: None}) == INVALID


@pytest.mark.parametrize("call,arg", [(fwd, "x"), (fwd, "y"), (bwd, "dw"), (lfwd, "z"), (lbwd, "dU")])
def test_misaligned_pointers(call, arg):
    assert call(**{arg: {"x": X, "y": Y, "dw": DW, "z": Z, "dU": DU}[arg] + 8}) == MISALIGNED


def test_channel_count_alignment():
    assert fwd(D=60, G=6) == MISALIGNED                  # bf16 rows must be 16-byte multiples
    assert fwd(D=60, G=6, dt=F32, y=X) == ALIASING       # fp32: a multiple of 4 is enough
    assert fwd(D=62, G=2, dt=F32) == MISALIGNED


def test_aliasing():
    # y on top of x (in place) is refused: later steps still read the old x
    assert fwd(y=X) == ALIASING
    # y overlapping the tail of w
    nbytes_w = 2 * 8 * 8 * 4 * 2
    assert fwd(y=Wp + nbytes_w - 16) == ALIASING
    assert bwd(dx=DY) == ALIASING
    assert bwd(dw=DX) == ALIASING                          # two outputs overlapping
    assert lbwd(dU=UU) == ALIASING
    assert lbwd(dz=DX) == ALIASING
    assert lbwd(ws=X) == ALIASING                          # workspace over an input


def test_too_large():
    assert fwd(D=1 << 25, G=1) == NOT_SUPPORTED


def test_workspace_query():
    L = dsc.lib()
    assert L.dsc_lowrank_bwd_workspace_bytes(0, 8, 64, 16, 4, BF16) == 0
    assert L.dsc_lowrank_bwd_workspace_bytes(2, 8, 64, 0, 4, BF16) == 0   # invalid -> 0
    for args in [(8, 4096, 2048, 32, 4), (1, 65536, 4096, 64, 8), (2, 100, 72, 24, 6)]:
        n = L.dsc_lowrank_bwd_workspace_bytes(*args, BF16)
        assert n % 16 == 0
        if n:
            assert lbwd(B=args[0], T=args[1], D=args[2], R=args[3], W=args[4], ws=None, wsb=0) == INVALID
            assert lbwd(B=args[0], T=args[1], D=args[2], R=args[3], W=args[4], ws=WS, wsb=n - 16) == WORKSPACE
            assert lbwd(B=args[0], T=args[1], D=args[2], R=args[3], W=args[4], ws=WS + 8, wsb=n) == MISALIGNED
            # an adequate workspace passes; the aliasing check (the last before a launch) then stops it
            assert lbwd(B=args[0], T=args[1], D=args[2], R=args[3], W=args[4], dU=UU, wsb=n) == ALIASING


# ------------------------------------------------------------------ decoding

POS, RING = A * 1500, A * 1600   # fake int32 positions and ring, far from the rest


def dec(x=X, w=Wp, pos=POS, state=RING, y=Y, B=4, D=64, G=8, W=4, res=1, dt=BF16):
    return dsc.lib().dsc_decode_step(x, w, pos, state, y, B, D, G, W, res, dt, None)


def ldec(x=X, z=Z, U=UU, pos=POS, state=RING, y=Y, B=4, D=64, R=16, W=4, res=0, dt=BF16):
    return dsc.lib().dsc_lowrank_decode_step(x, z, U, pos, state, y, B, D, R, W, res, dt, None)


def pre(x=X, ln=POS, state=RING, B=4, T=8, D=64, W=4, dt=BF16):
    return dsc.lib().dsc_decode_state_from_prefill(x, ln, state, B, T, D, W, dt, None)


def test_decode_empty_is_a_noop():
    assert dec(B=0) == OK and ldec(B=0) == OK and pre(B=0) == OK and pre(T=0) == OK
    assert dec(B=0, x=None, pos=None) == OK
    assert pre(W=1, state=None) == OK     # no ring to fill


@pytest.mark.parametrize("call", [dec, ldec])
def test_decode_invalid_values(call):
    assert call(B=-1) == INVALID
    assert call(D=0) == INVALID
    assert call(W=0) == INVALID
    assert call(W=9) == INVALID
    assert call(dt=5) == INVALID
    assert call(res=3) == INVALID
    assert call(x=None) == INVALID
    assert call(pos=None) == INVALID
    assert call(y=None) == INVALID
    assert call(state=None) == INVALID    # W > 1 needs a ring


def test_decode_specific_values():
    assert dec(G=0) == INVALID and dec(G=7) == INVALID and dec(w=None) == INVALID
    assert ldec(R=0) == INVALID and ldec(R=129) == INVALID and ldec(U=None) == INVALID
    assert pre(T=-1) == INVALID and pre(ln=None) == INVALID and pre(state=None) == INVALID


def test_decode_width_one_needs_no_ring():
    # state NULL passes validation when W == 1; y over x then stops the call before a launch
    assert dec(W=1, state=None, y=X) == ALIASING
    assert ldec(W=1, state=None, y=X) == ALIASING


def test_decode_alignment():
    assert dec(x=X + 8) == MISALIGNED
    assert dec(state=RING + 8) == MISALIGNED
    assert ldec(U=UU + 2) == MISALIGNED
    assert dec(pos=POS + 2) == MISALIGNED
    assert dec(pos=POS + 4, y=X) == ALIASING        # int32 positions need only 4-byte alignment
    assert dec(D=60, G=6) == MISALIGNED
    assert pre(ln=POS + 1) == MISALIGNED
    assert pre(state=RING + 4) == MISALIGNED


def test_decode_aliasing():
    assert dec(y=X) == ALIASING
    assert dec(state=X) == ALIASING                 # the ring over an input
    assert dec(state=Y) == ALIASING                 # the ring over y
    assert dec(state=POS - 16) == ALIASING          # the ring over the positions
    assert ldec(y=UU + 64) == ALIASING
    assert pre(state=X) == ALIASING
    assert pre(ln=RING + 16) == ALIASING


def test_decode_too_large():
    assert dec(D=1 << 25, G=1) == NOT_SUPPORTED
    assert dec(B=1 << 20, D=1 << 12, G=1 << 12) == NOT_SUPPORTED   # ring of 3 * 2^32 elements
    assert pre(B=1 << 20, T=1, D=1 << 12) == NOT_SUPPORTED


# ------------------------------------------------------------------ packed sequences

PP = A * 1700  # fake int32 positions


def vfwd(x=X, w=Wp, pos=PP, y=Y, B=2, T=8, D=64, G=8, W=4, res=1, dt=BF16):
    return dsc.lib().dsc_fwd_varlen(x, w, pos, y, B, T, D, G, W, res, dt, None)


def vbwd(x=X, w=Wp, pos=PP, dy=DY, dx=DX, dw=DW, B=2, T=8, D=64, G=8, W=4, res=1, dt=BF16):
    return dsc.lib().dsc_bwd_varlen(x, w, pos, dy, dx, dw, B, T, D, G, W, res, dt, None)


def vlfwd(x=X, z=Z, U=UU, pos=PP, y=Y, B=2, T=8, D=64, R=16, W=4, res=0, dt=BF16):
    return dsc.lib().dsc_lowrank_fwd_varlen(x, z, U, pos, y, B, T, D, R, W, res, dt, None)


def vlbwd(x=X, z=Z, U=UU, pos=PP, dy=DY, dx=DX, dz=DZ, dU=DU, ws=WS, wsb=1 << 40, B=2, T=8, D=64, R=16, W=4, res=0,
          dt=BF16):
    return dsc.lib().dsc_lowrank_bwd_varlen(x, z, U, pos, dy, dx, dz, dU, ws, wsb, B, T, D, R, W, res, dt, None)


@pytest.mark.parametrize("call", [vfwd, vbwd, vlfwd, vlbwd])
def test_varlen_checks(call):
    assert call(B=0) == OK and call(T=0) == OK
    assert call(B=-1) == INVALID and call(W=9) == INVALID and call(dt=3) == INVALID
    assert call(pos=None) == INVALID                 # positions are required
    assert call(pos=PP + 2) == MISALIGNED            # int32: 4-byte alignment
    assert call(pos=PP + 4, x=X + 8) == MISALIGNED   # tensors keep 16-byte alignment
    assert call(pos=PP + 4, **{("y" if call in (vfwd, vlfwd) else "dx"): PP}) == ALIASING  # an output over pos


def test_varlen_pos_alignment_passes_validation():
    # 4-byte aligned positions pass; the aliasing check (the last before a launch) then stops the call
    assert vfwd(pos=PP + 4, y=X) == ALIASING
    assert vlbwd(pos=PP + 4, dU=UU) == ALIASING


# ------------------------------------------------------------------ rotary epilogue

COS, SIN = A * 1800, A * 1900  # fake float32 tables


def rope(n_pos=64, d_rot=32, hd=16, inter=0, cos=COS, sin=SIN):
    return dsc.DscRope(cos, sin, n_pos, d_rot, hd, inter)


def rfwd(x=X, w=Wp, pos=None, r="default", y=Y, B=2, T=8, D=64, G=8, W=4, res=1, dt=BF16):
    r = rope() if r == "default" else r
    return dsc.lib().dsc_fwd_rope(x, w, pos, ctypes.byref(r) if r is not None else None, y, B, T, D, G, W, res, dt,
                                  None)


def rbwd(x=X, w=Wp, pos=None, r="default", dy=DY, dx=DX, dw=DW, B=2, T=8, D=64, G=8, W=4, res=1, dt=BF16):
    r = rope() if r == "default" else r
    return dsc.lib().dsc_bwd_rope(x, w, pos, ctypes.byref(r) if r is not None else None, dy, dx, dw, B, T, D, G, W,
                                  res, dt, None)


@pytest.mark.parametrize("call", [rfwd, rbwd])
def test_rope_checks(call):
    out = "y" if call is rfwd else "dx"
    assert call(B=0) == OK and call(T=0) == OK
    assert call(r=None) == INVALID
    assert call(r=rope(cos=None)) == INVALID
    assert call(r=rope(hd=8, d_rot=32)) == INVALID      # head size below 16
    assert call(r=rope(hd=48, d_rot=48)) == INVALID     # not a power of two
    assert call(r=rope(d_rot=24)) == INVALID            # not a multiple of the head size
    assert call(r=rope(d_rot=80)) == INVALID            # past D
    assert call(r=rope(inter=2)) == INVALID
    assert call(r=rope(n_pos=7)) == INVALID             # positions 0..7 without pos
    assert call(G=4, D=48) == NOT_SUPPORTED             # 12 channels per filter: no rotary layout
    assert call(r=rope(cos=COS + 8)) == MISALIGNED      # float4 reads of the tables
    # valid arguments reach the aliasing check, the last before a launch
    assert call(**{out: X}) == ALIASING
    assert call(r=rope(sin=Y if call is rfwd else DX)) == ALIASING        # an output over a table
    assert call(pos=PP, r=rope(n_pos=7), **{out: X}) == ALIASING         # with positions: clamped, no limit


# ------------------------------------------------------------------ generator in the kernel

HH, WG = A * 2000, A * 2100  # fake hidden state and generator weight


def gfwd(x=X, h=HH, wg=WG, y=Y, B=2, T=8, D=256, G=32, W=4, K=64, res=1, dt=BF16):
    return dsc.lib().dsc_fwd_gen(x, h, wg, y, B, T, D, G, W, K, res, dt, None)


def test_gen_checks():
    assert gfwd(B=0) == OK and gfwd(T=0) == OK
    assert gfwd(B=-1) == INVALID and gfwd(K=0) == INVALID and gfwd(h=None) == INVALID and gfwd(G=7) == INVALID
    assert gfwd(dt=F32) == NOT_SUPPORTED        # bf16 only
    assert gfwd(G=16, D=128) == NOT_SUPPORTED   # heads in blocks of 32
    assert gfwd(K=96) == NOT_SUPPORTED          # K in stages of 64
    assert gfwd(G=64, D=256) == NOT_SUPPORTED   # 4 channels per head: groups of 8 must sit in one head
    assert gfwd(h=HH + 8) == MISALIGNED
    assert gfwd(y=HH) == ALIASING               # valid arguments reach the aliasing check


def gfwd_var(x=X, h=HH, wg=WG, pos=PP, y=Y, B=2, T=8, D=256, G=32, W=4, K=64, res=1, dt=BF16):
    return dsc.lib().dsc_fwd_gen_varlen(x, h, wg, pos, y, B, T, D, G, W, K, res, dt, None)


def test_gen_varlen_checks():
    assert gfwd_var(B=0) == OK
    assert gfwd_var(pos=None) == INVALID        # positions are required
    assert gfwd_var(K=96) == NOT_SUPPORTED
    assert gfwd_var(pos=PP + 2) == MISALIGNED   # int32 positions
    assert gfwd_var(y=PP) == ALIASING           # the positions are an input
    assert gfwd_var(y=HH) == ALIASING


def gbwd(x=X, h=HH, wg=WG, dy=DY, dx=DX, dw=DW, B=2, T=8, D=256, G=32, W=4, K=64, res=1, dt=BF16):
    return dsc.lib().dsc_bwd_gen(x, h, wg, dy, dx, dw, B, T, D, G, W, K, res, dt, None)


def gbwd_var(x=X, h=HH, wg=WG, pos=PP, dy=DY, dx=DX, dw=DW, B=2, T=8, D=256, G=32, W=4, K=64, res=1, dt=BF16):
    return dsc.lib().dsc_bwd_gen_varlen(x, h, wg, pos, dy, dx, dw, B, T, D, G, W, K, res, dt, None)


def test_gen_bwd_checks():
    assert gbwd(B=0) == OK and gbwd(T=0, dw=None) == OK
    assert gbwd(B=-1) == INVALID and gbwd(W=0) == INVALID and gbwd(W=9) == INVALID
    assert gbwd(dw=None) == INVALID and gbwd(dy=None) == INVALID and gbwd(res=2) == INVALID
    assert gbwd(dt=F32) == NOT_SUPPORTED        # bf16 only
    assert gbwd(K=96) == NOT_SUPPORTED          # K in stages of 64
    assert gbwd(G=32, D=768) == NOT_SUPPORTED   # 24 channels per head: 3 groups of 8, not a power of two
    assert gbwd(G=32, D=8192) == NOT_SUPPORTED  # 256 channels per head: past 16 groups
    assert gbwd(G=32, D=4096, dx=DY) == ALIASING  # 128 channels per head: past the size checks
    assert gbwd(dw=DW + 4) == MISALIGNED and gbwd(dy=DY + 2) == MISALIGNED
    assert gbwd(dx=DY) == ALIASING and gbwd(dw=HH) == ALIASING and gbwd(dw=DX) == ALIASING
    assert gbwd_var(pos=None) == INVALID
    assert gbwd_var(pos=PP + 2) == MISALIGNED
    assert gbwd_var(dw=PP) == ALIASING


def lbwd_noalloc(x=X, z=Z, U=UU, dy=DY, dx=DX, dz=DZ, dU=DU, B=2, T=8, D=64, R=16, W=4, res=0, dt=BF16):
    return dsc.lib().dsc_lowrank_bwd_noalloc(x, z, U, dy, dx, dz, dU, B, T, D, R, W, res, dt, None)


def test_noalloc_checks():
    # the same checks as dsc_lowrank_bwd, in the same order, before anything is enqueued
    assert lbwd_noalloc(B=0) == OK
    assert lbwd_noalloc(B=0, x=None) == OK
    assert lbwd_noalloc(B=-1) == INVALID
    assert lbwd_noalloc(W=9) == INVALID
    assert lbwd_noalloc(R=0) == INVALID
    assert lbwd_noalloc(dt=7) == INVALID
    assert lbwd_noalloc(res=2) == INVALID
    assert lbwd_noalloc(dz=None) == INVALID
    assert lbwd_noalloc(dU=DU + 8) == MISALIGNED
    assert lbwd_noalloc(D=60) == MISALIGNED
    # a problem whose partial sums need more than the library's scratch array
    L = dsc.lib()
    assert L.dsc_lowrank_bwd_workspace_bytes(16, 4096, 2048, 32, 4, BF16) > dsc.NOALLOC_SCRATCH_BYTES
    assert lbwd_noalloc(B=16, T=4096, D=2048, R=32, W=4) == WORKSPACE
    # within the array, aliasing is still refused
    assert L.dsc_lowrank_bwd_workspace_bytes(8, 4096, 2048, 32, 4, BF16) <= dsc.NOALLOC_SCRATCH_BYTES
    assert lbwd_noalloc(dz=DX) == ALIASING
    assert lbwd_noalloc(dU=UU) == ALIASING
