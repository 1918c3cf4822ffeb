"""Parity of the packed-sequence entry points (dsc_fwd_varlen, dsc_bwd_varlen,
dsc_lowrank_fwd_varlen, dsc_lowrank_bwd_varlen) with the CPU oracle.

Rows pack sequences of random lengths (1, shorter than W, long), with pos[b,t]
the index of each token within its sequence. Small shapes: every output element
against the oracle with the same positions. Positions equal to t reproduce the
dense kernels bit for bit. A NaN planted in one sequence leaves every other
sequence's outputs bitwise unchanged (the masks select, they do not multiply).
The packed workloads at full size: sampled tokens (and dU columns) against the
oracle. Tolerance: max |gpu - ref| <= tol * (1 + |ref|).
"""
import zlib

import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
import oracle
from dynamic_short_convolutions_amd.synthetic import WORKLOADS, Workload, draw, packed_positions
from gpu_helpers import TOL, assert_close, check_guard, dev, host, poisoned, sample_rows, torch

pytestmark = pytest.mark.gpu


def ipos(p):
    return torch().from_numpy(np.ascontiguousarray(p, dtype=np.int32)).cuda()


def workspace_for(x, R, W):
    t = torch()
    B, T, D = x.shape
    code = dsc.DSC_BF16 if x.dtype == t.bfloat16 else dsc.DSC_F32
    n = dsc.dsc_lowrank_bwd_workspace_bytes(B, T, D, R, W, code)
    return t.full((max(n, 16),), 0xFF, dtype=t.uint8, device="cuda") if n else None


def run_headwise(x, w, pos, dy, res):
    y, yb = poisoned(tuple(x.shape), x.dtype)
    dx, dxb = poisoned(tuple(x.shape), x.dtype)
    dw, dwb = poisoned(tuple(w.shape), x.dtype)
    dsc.dsc_fwd_varlen(x, w, pos, y, res)
    dsc.dsc_bwd_varlen(x, w, pos, dy, dx, dw, res)
    torch().cuda.synchronize()
    for buf, o, n in ((yb, y, "y"), (dxb, dx, "dx"), (dwb, dw, "dw")):
        check_guard(buf, o.numel(), n)
    return y, dx, dw


def run_lowrank(x, z, U, pos, dy, W, res):
    y, yb = poisoned(tuple(x.shape), x.dtype)
    dx, dxb = poisoned(tuple(x.shape), x.dtype)
    dz, dzb = poisoned(tuple(z.shape), x.dtype)
    dU, dUb = poisoned(tuple(U.shape), x.dtype)
    dsc.dsc_lowrank_fwd_varlen(x, z, U, pos, y, W, res)
    dsc.dsc_lowrank_bwd_varlen(x, z, U, pos, dy, dx, dz, dU, workspace_for(x, z.shape[2], W), W, res)
    torch().cuda.synchronize()
    for buf, o, n in ((yb, y, "y"), (dxb, dx, "dx"), (dzb, dz, "dz"), (dUb, dU, "dU")):
        check_guard(buf, o.numel(), n)
    return y, dx, dz, dU


# (kind, B, T, D, Hc or R, W, residual, dtype, mean sequence length)
CASES = [
    ("headwise", 2, 300, 1024, 8, 4, 1, "bf16", 20),
    ("headwise", 2, 129, 1024, 16, 4, 1, "bf16", 6),     # heads spanning lanes, many short sequences
    ("headwise", 1, 200, 96, 1, 8, 1, "bf16", 5),        # per-channel filters, 8 taps
    ("headwise", 2, 130, 1088, 1, 4, 0, "bf16", 7),      # per-channel filters, taps through LDS, partial wave
    ("headwise", 2, 150, 72, 24, 6, 0, "bf16", 9),       # generic head size: dw by its own kernel
    ("headwise", 1, 60, 2400, 24, 4, 1, "f32", 7),       # ... 100 heads: dw over two blocks of 64 heads
    ("headwise", 2, 120, 1440, 12, 4, 1, "bf16", 6),     # 120 heads of 12: dw from 4-channel groups
    ("headwise", 3, 97, 40, 4, 7, 1, "f32", 4),
    ("headwise", 2, 64, 48, 2, 2, 0, "f32", 3),
    ("headwise", 1, 100, 8, 8, 1, 1, "bf16", 3),         # W = 1: positions change nothing
    ("lowrank", 2, 300, 256, 32, 4, 0, "bf16", 25),      # fused dz
    ("lowrank", 2, 200, 128, 64, 8, 1, "bf16", 7),       # separate dz pass, tap-split dx+dU
    ("lowrank", 1, 257, 192, 16, 3, 1, "bf16", 4),
    ("lowrank", 2, 130, 64, 128, 6, 0, "bf16", 12),
    ("lowrank", 2, 150, 128, 16, 3, 1, "bf16", 9),       # forward with time in the lane, three taps
    ("lowrank", 2, 90, 40, 5, 4, 1, "bf16", 6),          # vector kernels (R % 8 != 0)
    ("lowrank", 2, 70, 24, 4, 5, 0, "f32", 5),           # fp32: vector kernels
    ("lowrank", 3, 237, 152, 64, 4, 1, "f32", 33),       # fp32, long dU sums
]
LOWRANK_CASES = [c for c in CASES if c[0] == "lowrank"]  # the first: fused dz; the second: its own dz pass


def _inputs(case):
    kind, B, T, D, HR, W, res, dt, mean = case
    seed = zlib.crc32(repr(case).encode())
    if kind == "headwise":
        wl = Workload("var_hw", kind, B=B, T=T, D=D, W=W, residual=res, dtype=dt, Hc=HR)
    else:
        wl = Workload("var_lr", kind, B=B, T=T, D=D, W=W, residual=res, dtype=dt, R=HR, U_std=1.0 / np.sqrt(HR * W))
    inp = draw(wl, seed=seed, need_dy=True)
    inp["pos"] = packed_positions(B, T, mean, seed + 7)
    return inp


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{}_B{}T{}D{}_{}W{}r{}{}_L{}".format(*c))
def test_varlen_parity_small(case):
    kind, B, T, D, HR, W, res, dt, mean = case
    inp = _inputs(case)
    pos = inp["pos"]
    tol = TOL[dt]
    if kind == "headwise":
        y, dx, dw = run_headwise(dev(inp["x"]), dev(inp["w"]), ipos(pos), dev(inp["dy"]), res)
        assert_close(host(y), oracle.fwd(inp["x"], inp["w"], res, pos=pos), tol, "y")
        dx_ref, dw_ref = oracle.bwd(inp["x"], inp["w"], inp["dy"], res, pos=pos)
        assert_close(host(dx), dx_ref, tol, "dx")
        assert_close(host(dw), dw_ref, tol, "dw")
    else:
        y, dx, dz, dU = run_lowrank(dev(inp["x"]), dev(inp["z"]), dev(inp["U"]), ipos(pos), dev(inp["dy"]), W, res)
        assert_close(host(y), oracle.lowrank_fwd(inp["x"], inp["z"], inp["U"], W, res, pos=pos), tol, "y")
        dx_ref, dz_ref, dU_ref = oracle.lowrank_bwd(inp["x"], inp["z"], inp["U"], inp["dy"], W, res, pos=pos)
        assert_close(host(dx), dx_ref, tol, "dx")
        assert_close(host(dz), dz_ref, tol, "dz")
        assert_close(host(dU), dU_ref, tol, "dU")


@pytest.mark.parametrize("case", [CASES[0], CASES[1], LOWRANK_CASES[0], LOWRANK_CASES[1]], ids=lambda c: f"{c[0]}_W{c[5]}")
def test_positions_from_zero_equal_dense_bitwise(case):
    """pos[b,t] = t: every tap exists, and the varlen kernels give the dense bits."""
    kind, B, T, D, HR, W, res, dt, mean = case
    t = torch()
    inp = _inputs(case)
    pos = ipos(np.tile(np.arange(T, dtype=np.int32), (B, 1)))
    if kind == "headwise":
        x, w, dy = dev(inp["x"]), dev(inp["w"]), dev(inp["dy"])
        got = run_headwise(x, w, pos, dy, res)
        y, dx, dw = t.empty_like(x), t.empty_like(x), t.empty_like(w)
        dsc.dsc_fwd(x, w, y, res)
        dsc.dsc_bwd(x, w, dy, dx, dw, res)
        ref = (y, dx, dw)
    else:
        x, z, U, dy = dev(inp["x"]), dev(inp["z"]), dev(inp["U"]), dev(inp["dy"])
        got = run_lowrank(x, z, U, pos, dy, W, res)
        y, dx, dz, dU = t.empty_like(x), t.empty_like(x), t.empty_like(z), t.empty_like(U)
        dsc.dsc_lowrank_fwd(x, z, U, y, W, res)
        dsc.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, workspace_for(x, z.shape[2], W), W, res)
        ref = (y, dx, dz, dU)
    t.cuda.synchronize()
    for a, b in zip(got, ref):
        assert t.equal(a.view(t.int16), b.view(t.int16))


@pytest.mark.parametrize("kind", ["headwise", "lowrank"])
def test_nan_stays_in_its_sequence(kind):
    """A NaN in one sequence's x and dy changes no output of any other sequence."""
    t = torch()
    case = CASES[0] if kind == "headwise" else LOWRANK_CASES[0]
    _, B, T, D, HR, W, res, dt, mean = case
    inp = _inputs(case)
    pos = inp["pos"]
    starts = np.flatnonzero(pos[0] == 0)
    s0, s1 = int(starts[2]), int(starts[3])  # the third sequence of row 0
    x2, dy2 = inp["x"].copy(), inp["dy"].copy()
    x2[0, s0:s1, :5] = 0x7FC0  # bf16 NaN
    dy2[0, s0:s1, 3:9] = 0x7FC0
    other = np.ones((B, T), bool)
    other[0, s0:s1] = False
    if kind == "headwise":
        a = run_headwise(dev(inp["x"]), dev(inp["w"]), ipos(pos), dev(inp["dy"]), res)
        b = run_headwise(dev(x2), dev(inp["w"]), ipos(pos), dev(dy2), res)
    else:
        a = run_lowrank(dev(inp["x"]), dev(inp["z"]), dev(inp["U"]), ipos(pos), dev(inp["dy"]), W, res)[:3]
        b = run_lowrank(dev(x2), dev(inp["z"]), dev(inp["U"]), ipos(pos), dev(dy2), W, res)[:3]
    m = t.from_numpy(other).cuda()
    for u, v in zip(a, b):
        assert t.equal(u[m].view(t.int16), v[m].view(t.int16))
    assert bool(t.isnan(b[0][0, s0:s1].float()).any())  # and the NaN did reach its own sequence


@pytest.mark.parametrize("name", ["packed_qkv_headwise_bf16", "packed_lowrank_bf16"])
def test_packed_workloads_full_size(name):
    """Full sizes, default launch configuration; the oracle on sampled tokens (and dU columns)."""
    wl = WORKLOADS[name]
    print(f"[{name}] drawing inputs", flush=True)
    inp = draw(wl)
    pos = inp["pos"]
    x, dy = dev(inp["x"]), dev(inp["dy"])
    # sampled tokens: sequence starts and their neighbours, plus the usual tile edges
    st = np.flatnonzero(pos.reshape(-1) == 0)
    rows = np.unique(np.concatenate([sample_rows(wl.B, wl.T, n_random=30, seed=6),
                                     np.clip(np.concatenate([st, st + 1, st + 2, st + 3, st - 1]), 0,
                                             wl.B * wl.T - 1)[:400]]))
    flat = lambda t, n: host(t.reshape(wl.B * wl.T, n)[torch().from_numpy(rows).cuda()])
    tol = TOL[wl.dtype]
    if wl.kind == "headwise":
        print(f"[{name}] GPU", flush=True)
        y, dx, dw = run_headwise(x, dev(inp["w"]), ipos(pos), dy, wl.residual)
        print(f"[{name}] oracle on {rows.size} tokens", flush=True)
        assert_close(flat(y, wl.D), oracle.fwd(inp["x"], inp["w"], wl.residual, rows=rows, pos=pos), tol, "y")
        dx_ref, dw_ref = oracle.bwd(inp["x"], inp["w"], inp["dy"], wl.residual, rows=rows, pos=pos)
        assert_close(flat(dx, wl.D), dx_ref, tol, "dx")
        assert_close(flat(dw, wl.G * wl.W).reshape(-1, wl.G, wl.W), dw_ref, tol, "dw")
    else:
        print(f"[{name}] GPU", flush=True)
        y, dx, dz, dU = run_lowrank(x, dev(inp["z"]), dev(inp["U"]), ipos(pos), dy, wl.W, wl.residual)
        print(f"[{name}] oracle on {rows.size} tokens", flush=True)
        assert_close(flat(y, wl.D), oracle.lowrank_fwd(inp["x"], inp["z"], inp["U"], wl.W, wl.residual,
                                                       rows=rows, pos=pos), tol, "y")
        dx_ref, dz_ref = oracle.lowrank_bwd_rows(inp["x"], inp["z"], inp["U"], inp["dy"], wl.W, wl.residual,
                                                 rows=rows, pos=pos)
        assert_close(flat(dx, wl.D), dx_ref, tol, "dx")
        assert_close(flat(dz, wl.R), dz_ref, tol, "dz")
        cols = np.random.default_rng(8).choice(wl.D * wl.W, size=24, replace=False)
        dU_ref = oracle.lowrank_dU(inp["x"], inp["z"], inp["dy"], wl.W, cols=cols, pos=pos)
        assert_close(host(dU)[:, cols], dU_ref, tol, "dU")
