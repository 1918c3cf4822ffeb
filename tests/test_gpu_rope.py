"""Parity of the fused rotary epilogue (dsc_fwd_rope, dsc_bwd_rope) with the CPU oracle.

The oracle composes the head-wise convolution with the rotary embedding of its
first d_rot channels (and, for the backward, takes dy back through the
transposed rotation). Small shapes: every element, both pairings, head sizes
16 to 512 (partner lanes 1 to 32 apart), filter layouts in a lane and across
lanes, fp32 and bf16, dense and packed positions. d_rot = 0 gives the dense
kernels' bits. The QKV workload with the rotary epilogue at full size on
sampled tokens. Tolerance: max |gpu - ref| <= tol * (1 + |ref|).
"""
import zlib

import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
import oracle
from dynamic_short_convolutions_amd.synthetic import WORKLOADS, Workload, draw, packed_positions, rope_table
from gpu_helpers import TOL, assert_close, check_guard, dev, host, poisoned, sample_rows, torch

pytestmark = pytest.mark.gpu


def ipos(p):
    return None if p is None else torch().from_numpy(np.ascontiguousarray(p, dtype=np.int32)).cuda()


def run(x, w, pos, tables, d_rot, hd, inter, dy, res):
    cos, sin = (torch().from_numpy(t).cuda() for t in tables)
    r = dsc.rope_args(cos, sin, d_rot, hd, inter)
    y, yb = poisoned(tuple(x.shape), x.dtype)
    dx, dxb = poisoned(tuple(x.shape), x.dtype)
    dw, dwb = poisoned(tuple(w.shape), x.dtype)
    dsc.dsc_fwd_rope(x, w, pos, r, y, res)
    dsc.dsc_bwd_rope(x, w, pos, r, dy, dx, dw, res)
    torch().cuda.synchronize()
    for buf, o, n in ((yb, y, "y"), (dxb, dx, "dx"), (dwb, dw, "dw")):
        check_guard(buf, o.numel(), n)
    return y, dx, dw


# (B, T, D, Hc, W, residual, dtype, head_dim, d_rot, interleaved, packed mean length or 0)
CASES = [
    (2, 150, 384, 8, 4, 1, "bf16", 64, 256, 0, 0),      # Q, K rotated, V passes
    (2, 150, 384, 8, 4, 1, "bf16", 64, 256, 1, 0),      # interleaved pairs
    (1, 100, 1024, 16, 4, 1, "bf16", 128, 512, 0, 0),   # filter heads across lanes
    (2, 77, 512, 1, 3, 0, "bf16", 512, 512, 0, 0),      # largest head: partners 32 lanes apart
    (2, 90, 64, 2, 5, 1, "bf16", 16, 64, 0, 0),         # smallest head, all channels rotated
    (2, 90, 64, 4, 8, 0, "f32", 16, 32, 0, 0),
    (1, 64, 256, 8, 2, 1, "f32", 32, 128, 1, 0),
    (2, 200, 384, 8, 4, 1, "bf16", 64, 256, 0, 12),     # packed sequences: positions restart
    (2, 130, 256, 32, 6, 0, "bf16", 128, 256, 1, 7),
    (3, 33, 128, 8, 4, 1, "bf16", 32, 64, 0, 0),        # three sequences, ragged tiles
]


def _inputs(case):
    B, T, D, Hc, W, res, dt, hd, d_rot, inter, packed = case
    seed = zlib.crc32(repr(case).encode())
    wl = Workload("rope", "headwise", B=B, T=T, D=D, W=W, residual=res, dtype=dt, Hc=Hc)
    inp = draw(wl, seed=seed, need_dy=True)
    pos = packed_positions(B, T, packed, seed + 3) if packed else None
    return inp, pos, rope_table(T + 5, hd)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}D{}Hc{}W{}r{}{}_hd{}_rot{}_i{}_p{}".format(*c))
def test_rope_parity_small(case):
    B, T, D, Hc, W, res, dt, hd, d_rot, inter, packed = case
    inp, pos, tables = _inputs(case)
    y, dx, dw = run(dev(inp["x"]), dev(inp["w"]), ipos(pos), tables, d_rot, hd, inter, dev(inp["dy"]), res)
    cos, sin = tables
    tol = TOL[dt]
    assert_close(host(y), oracle.fwd_rope(inp["x"], inp["w"], res, cos, sin, d_rot, hd, inter, pos=pos), tol, "y")
    dx_ref, dw_ref = oracle.bwd_rope(inp["x"], inp["w"], inp["dy"], res, cos, sin, d_rot, hd, inter, pos=pos)
    assert_close(host(dx), dx_ref, tol, "dx")
    assert_close(host(dw), dw_ref, tol, "dw")


@pytest.mark.parametrize("packed", [0, 9])
def test_nothing_rotated_is_the_plain_convolution(packed):
    """d_rot = 0: the rotary instances give the bits of dsc_fwd/dsc_bwd (or the _varlen pair)."""
    t = torch()
    case = (2, 150, 384, 8, 4, 1, "bf16", 64, 0, 0, packed)
    inp, pos, tables = _inputs(case)
    x, w, dy = dev(inp["x"]), dev(inp["w"]), dev(inp["dy"])
    got = run(x, w, ipos(pos), tables, 0, 64, 0, dy, 1)
    y, dx, dw = t.empty_like(x), t.empty_like(x), t.empty_like(w)
    if pos is None:
        dsc.dsc_fwd(x, w, y, 1)
        dsc.dsc_bwd(x, w, dy, dx, dw, 1)
    else:
        dsc.dsc_fwd_varlen(x, w, ipos(pos), y, 1)
        dsc.dsc_bwd_varlen(x, w, ipos(pos), dy, dx, dw, 1)
    t.cuda.synchronize()
    for a, b in zip(got, (y, dx, dw)):
        assert t.equal(a.view(t.int16), b.view(t.int16))


def test_rope_workload_full_size():
    wl = WORKLOADS["rope_qkv_headwise_bf16"]
    print(f"[{wl.name}] drawing inputs", flush=True)
    inp = draw(wl)
    tables = rope_table(wl.T, wl.rope_head_dim)
    print(f"[{wl.name}] GPU", flush=True)
    y, dx, dw = run(dev(inp["x"]), dev(inp["w"]), None, tables, wl.rope_d_rot, wl.rope_head_dim,
                    wl.rope_interleaved, dev(inp["dy"]), wl.residual)
    rows = sample_rows(wl.B, wl.T, n_random=40, seed=5)
    flat = lambda t, n: host(t.reshape(wl.B * wl.T, n)[torch().from_numpy(rows).cuda()])
    cos, sin = tables
    tol = TOL[wl.dtype]
    print(f"[{wl.name}] oracle on {rows.size} tokens", flush=True)
    y_ref = oracle.fwd_rope(inp["x"], inp["w"], wl.residual, cos, sin, wl.rope_d_rot, wl.rope_head_dim,
                            wl.rope_interleaved, rows=rows)
    assert_close(flat(y, wl.D), y_ref, tol, "y")
    dx_ref, dw_ref = oracle.bwd_rope(inp["x"], inp["w"], inp["dy"], wl.residual, cos, sin, wl.rope_d_rot,
                                     wl.rope_head_dim, wl.rope_interleaved, rows=rows)
    assert_close(flat(dx, wl.D), dx_ref, tol, "dx")
    assert_close(flat(dw, wl.G * wl.W).reshape(-1, wl.G, wl.W), dw_ref, tol, "dw")
