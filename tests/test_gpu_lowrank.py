"""Parity of the low-rank HIP kernels (dsc_lowrank_fwd, dsc_lowrank_bwd) with the CPU oracle.

Small shapes: every output element. Full-size workloads (the benchmark's launch
configuration): sampled tokens for y, dx and dz, sampled columns of dU (each the
sum over every token), plus all-written, guard-band and bit-for-bit
repeatability checks. Tolerance: max |gpu - ref| <= tol * (1 + |ref|).
"""
import zlib

import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
import oracle
from dynamic_short_convolutions_amd.synthetic import WORKLOADS, Workload, draw
from gpu_helpers import TOL, assert_close, check_guard, dev, host, poisoned, sample_rows, torch

pytestmark = pytest.mark.gpu


def lowrank_case(B, T, D, R, W, res, dt):
    return Workload(f"lr_{B}x{T}x{D}_R{R}_W{W}_{dt}", "lowrank", B=B, T=T, D=D, W=W, residual=res,
                    dtype=dt, R=R, U_std=1.0 / np.sqrt(R * W))


def gpu_fwd(x, z, U, W, res):
    y, ybuf = poisoned(tuple(x.shape), x.dtype)
    dsc.dsc_lowrank_fwd(x, z, U, y, W, res)
    torch().cuda.synchronize()
    check_guard(ybuf, y.numel(), "y")
    return y


def workspace_for(x, R, W):
    t = torch()
    B, T, D = x.shape
    code = dsc.DSC_BF16 if x.dtype == t.bfloat16 else dsc.DSC_F32
    n = dsc.dsc_lowrank_bwd_workspace_bytes(B, T, D, R, W, code)
    # poisoned workspace: its contents on entry must not matter
    return t.full((max(n, 16),), 0xFF, dtype=t.uint8, device="cuda") if n else None


def gpu_bwd(x, z, U, dy, W, res, ws=None):
    t = torch()
    R = z.shape[2]
    dx, dxb = poisoned(tuple(x.shape), x.dtype)
    dz, dzb = poisoned(tuple(z.shape), x.dtype)
    dU, dUb = poisoned(tuple(U.shape), x.dtype)
    if ws is None:
        ws = workspace_for(x, R, W)
    dsc.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, ws, W, res)
    t.cuda.synchronize()
    for buf, o, n in ((dxb, dx, "dx"), (dzb, dz, "dz"), (dUb, dU, "dU")):
        check_guard(buf, o.numel(), n)
    return dx, dz, dU


CASES = [
    # (B, T, D, R, W, residual, dtype)
    (2, 300, 256, 32, 4, 0, "bf16"),     # the low-rank workload's R and W, several tiles, ragged T
    (1, 200, 128, 64, 8, 0, "bf16"),     # the long-sequence workload's R and W
    (2, 77, 520, 16, 4, 1, "bf16"),      # R below one MFMA step, ragged D
    (1, 129, 64, 40, 6, 1, "bf16"),      # R not a multiple of 32, 6 taps
    (2, 33, 24, 8, 2, 0, "bf16"),
    (1, 50, 16, 24, 3, 1, "bf16"),       # odd tap count
    (2, 9, 32, 128, 8, 0, "bf16"),       # maximum rank
    (1, 3, 16, 32, 4, 1, "bf16"),        # T < W
    (1, 1, 8, 8, 8, 0, "bf16"),          # T = 1
    (1, 90, 48, 16, 5, 0, "bf16"),       # odd tap counts pad the (channel, tap) pairs of dz
    (2, 64, 40, 32, 7, 1, "bf16"),
    (1, 45, 24, 8, 1, 1, "bf16"),        # one tap
    (1, 40, 256, 72, 8, 0, "bf16"),      # three K-steps of the filter, several forward channel blocks
    (1, 33, 192, 128, 6, 1, "bf16"),     # largest rank with six taps, several channel blocks
    (2, 77, 200, 48, 4, 0, "bf16"),      # separate dz pass, last 16-channel chunk half empty
    (1, 100, 192, 32, 3, 1, "bf16"),     # forward with time in the lane: W = 3, the block's last wave past D
    (2, 70, 128, 64, 2, 0, "bf16"),      # ... two K-steps of the filter (W = 2)
    (1, 50, 320, 128, 1, 1, "bf16"),     # ... four K-steps (W = 1), a second channel block of one wave
    (1, 37, 64, 16, 4, 1, "bf16"),       # ... one wave's channels, T not a multiple of 16
    (3, 16, 64, 8, 4, 0, "bf16"),        # ... T = 16, the smallest rank
    (2, 150, 96, 96, 4, 1, "bf16"),      # dx+dU with the taps split over two waves, partial channel block
    (1, 70, 40, 80, 6, 0, "bf16"),       # tap halves of three, ragged D
    (1, 100, 64, 48, 8, 1, "bf16"),      # tap halves of four
    (1, 60, 40, 12, 3, 1, "bf16"),       # bf16 rank not a multiple of 8: the vector kernels
    (2, 33, 16, 3, 5, 0, "bf16"),
    (2, 100, 36, 5, 4, 1, "f32"),        # fp32, D % 8 == 4
    (1, 70, 64, 32, 8, 0, "f32"),
    (3, 40, 8, 1, 1, 1, "f32"),          # rank 1, W = 1
    # fp32 dU and dz summed over a few hundred tokens whose partial sums cancel: an fp32
    # running sum missed the fp32 tolerance here; the vector kernels now sum in double
    (2, 251, 160, 64, 7, 0, "f32"),
    (2, 257, 228, 16, 2, 0, "f32"),
]


def _random_cases(n, seed):
    """Seeded random shapes across the launch plan's branches (fused dz for R <= 32, tap
    halves, rank tiles 1..8, vector kernels for fp32 and other ranks), sized for the oracle."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dt = "f32" if rng.random() < 0.2 else "bf16"
        R = int(rng.choice([8, 16, 24, 32, 40, 48, 64, 80, 96, 112, 128, 12, 5]))
        W = int(rng.integers(1, 9))
        D = int(rng.choice([8, 4]) if dt == "f32" else 8) * int(rng.integers(1, 70))
        T = int(rng.integers(1, 260))
        out.append((int(rng.integers(1, 3)), T, D, R, W, int(rng.integers(0, 2)), dt))
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(24, 91), ids=lambda c: "B{}T{}D{}R{}W{}r{}{}".format(*c))
def test_lowrank_parity_small(case):
    B, T, D, R, W, res, dt = case
    wl = lowrank_case(B, T, D, R, W, res, dt)
    inp = draw(wl, seed=zlib.crc32(repr(case).encode()), need_dy=True)
    x, z, U, dy = (dev(inp[k]) for k in ("x", "z", "U", "dy"))
    y = gpu_fwd(x, z, U, W, res)
    dx, dz, dU = gpu_bwd(x, z, U, dy, W, res)
    tol = TOL[dt]
    assert_close(host(y), oracle.lowrank_fwd(inp["x"], inp["z"], inp["U"], W, res), tol, "y")
    dx_r, dz_r, dU_r = oracle.lowrank_bwd(inp["x"], inp["z"], inp["U"], inp["dy"], W, res)
    assert_close(host(dx), dx_r, tol, "dx")
    assert_close(host(dz), dz_r, tol, "dz")
    assert_close(host(dU), dU_r, tol, "dU")


def test_vector_dU_past_its_capped_grid():
    """fp32 with 2^20 + 48 channels: the vector-ALU dU kernel's grid is capped at 2^16
    blocks of 16 channels, so its blocks stride over a second column block (the last
    one partial); every output element against the oracle."""
    B, T, D, R, W, res, dt = 1, 3, (1 << 20) + 48, 8, 2, 1, "f32"
    wl = lowrank_case(B, T, D, R, W, res, dt)
    inp = draw(wl, seed=77, need_dy=True)
    x, z, U, dy = (dev(inp[k]) for k in ("x", "z", "U", "dy"))
    print(f"[vector dU past the capped grid] D={D}", flush=True)
    dx, dz, dU = gpu_bwd(x, z, U, dy, W, res)
    dx_r, dz_r, dU_r = oracle.lowrank_bwd(inp["x"], inp["z"], inp["U"], inp["dy"], W, res)
    assert_close(host(dx), dx_r, TOL[dt], "dx")
    assert_close(host(dz), dz_r, TOL[dt], "dz")
    assert_close(host(dU), dU_r, TOL[dt], "dU")


@pytest.mark.parametrize("name", ["lowrank_bf16", "longseq_lowrank_bf16", "lowrank_f32"])
def test_full_size_workloads(name):
    wl = WORKLOADS[name]
    print(f"[{name}] drawing inputs", flush=True)
    inp = draw(wl)
    x, z, U, dy = (dev(inp[k]) for k in ("x", "z", "U", "dy"))
    print(f"[{name}] forward", flush=True)
    y = gpu_fwd(x, z, U, wl.W, wl.residual)
    print(f"[{name}] backward", flush=True)
    ws = workspace_for(x, wl.R, wl.W)
    dx, dz, dU = gpu_bwd(x, z, U, dy, wl.W, wl.residual, ws)
    tol = TOL[wl.dtype]
    rows = sample_rows(wl.B, wl.T, n_random=24, seed=6)
    idx = torch().from_numpy(rows).cuda()
    print(f"[{name}] oracle on {rows.size} sampled tokens", flush=True)
    assert_close(host(y.reshape(-1, wl.D)[idx]),
                 oracle.lowrank_fwd(inp["x"], inp["z"], inp["U"], wl.W, wl.residual, rows=rows), tol, "y")
    dx_r, dz_r = oracle.lowrank_bwd_rows(inp["x"], inp["z"], inp["U"], inp["dy"], wl.W, wl.residual, rows=rows)
    assert_close(host(dx.reshape(-1, wl.D)[idx]), dx_r, tol, "dx")
    assert_close(host(dz.reshape(-1, wl.R)[idx]), dz_r, tol, "dz")
    rng = np.random.default_rng(7)
    ncol = wl.D * wl.W
    cols = np.unique(np.concatenate([[0, 1, wl.W - 1, ncol - 1, ncol - wl.W],
                                     rng.integers(0, ncol, size=40)])).astype(np.int64)
    print(f"[{name}] oracle on {cols.size} sampled columns of dU", flush=True)
    dU_r = oracle.lowrank_dU(inp["x"], inp["z"], inp["dy"], wl.W, cols=cols)
    assert_close(host(dU[:, torch().from_numpy(cols).cuda()]), dU_r, tol, "dU")
    for t, n in ((y, "y"), (dx, "dx"), (dz, "dz"), (dU, "dU")):
        assert bool(torch().isfinite(t).all()), f"{n}: unwritten elements"
    y2 = gpu_fwd(x, z, U, wl.W, wl.residual)
    dx2, dz2, dU2 = gpu_bwd(x, z, U, dy, wl.W, wl.residual, ws)
    assert torch().equal(y, y2) and torch().equal(dx, dx2)
    assert torch().equal(dz, dz2) and torch().equal(dU, dU2)


def test_lowrank_equals_materialised_headwise_on_device():
    """The fused low-rank forward equals the head-wise forward (one channel per head)
    on filters z.U written out to memory by torch (fp32, exact for these integers)."""
    t = torch()
    g = t.Generator(device="cpu").manual_seed(3)
    B, T, D, R, W = 2, 90, 64, 16, 4
    x = t.randint(-2, 3, (B, T, D), generator=g).float()
    z = t.randint(-2, 3, (B, T, R), generator=g).float()
    U = t.randint(-2, 3, (R, D * W), generator=g).float()
    w = (z.reshape(B * T, R) @ U).reshape(B, T, D, W)
    xd, zd, Ud, wd = (a.cuda() for a in (x, z, U, w))
    y_lr = gpu_fwd(xd, zd, Ud, W, 1)
    y_hw, _ = poisoned((B, T, D), t.float32)
    dsc.dsc_fwd(xd, wd.contiguous(), y_hw, 1)
    t.cuda.synchronize()
    assert t.equal(y_lr, y_hw)
