"""Parity of the head-wise HIP kernels (dsc_fwd, dsc_bwd) with the CPU oracle.

Small shapes are compared element by element on every output; the full-size
workloads (the launch configuration the benchmark times) on sampled tokens,
plus properties that hold at any size: every output element is written, no
write lands past an output's end, and repeated calls agree bit for bit.
Tolerance: max |gpu - ref| <= tol * (1 + |ref|), tol 1e-5 (fp32) / 1e-2 (bf16).
"""
import zlib

import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
import oracle
from dynamic_short_convolutions_amd.synthetic import WORKLOADS, Workload, draw
from gpu_helpers import TOL, assert_close, check_guard, dev, host, poisoned, sample_rows, torch

pytestmark = pytest.mark.gpu


def headwise_case(B, T, D, Hc, W, res, dt, seed):
    return Workload(f"hw_{B}x{T}x{D}_Hc{Hc}_W{W}_{dt}", "headwise", B=B, T=T, D=D, W=W, residual=res,
                    dtype=dt, Hc=Hc), seed


def gpu_fwd(x, w, res):
    y, ybuf = poisoned(tuple(x.shape), x.dtype)
    dsc.dsc_fwd(x, w, y, res)
    torch().cuda.synchronize()
    check_guard(ybuf, y.numel(), "y")
    return y


def gpu_bwd(x, w, dy, res):
    dx, dxbuf = poisoned(tuple(x.shape), x.dtype)
    dw, dwbuf = poisoned(tuple(w.shape), x.dtype)
    dsc.dsc_bwd(x, w, dy, dx, dw, res)
    torch().cuda.synchronize()
    check_guard(dxbuf, dx.numel(), "dx")
    check_guard(dwbuf, dw.numel(), "dw")
    return dx, dw


# (B, T, D, Hc, W, residual, dtype): chosen to cover every head layout, several
# channel blocks and step tiles with ragged tails, every tap count, T < W, T = 1.
CASES = [
    (1, 256, 64, 8, 4, 1, "f32"),        # the tiny workload's shape
    (2, 300, 2056, 8, 4, 1, "bf16"),     # 2 channel blocks (257 groups), 5+ step tiles, ragged
    (2, 129, 1024, 16, 4, 1, "bf16"),    # a head spans 2 lanes
    (1, 70, 512, 32, 3, 0, "bf16"),      # 4 lanes per head, 3 taps (6-byte filters)
    (2, 64, 8192, 512, 4, 1, "bf16"),    # 64 lanes per head (a whole wave)
    (3, 33, 96, 1, 8, 1, "bf16"),        # per-channel filters, 8 taps
    (2, 17, 48, 2, 2, 0, "f32"),         # 4 heads per group
    (2, 65, 40, 4, 5, 1, "f32"),         # 2 heads per group, 5 taps
    (1, 40, 12, 4, 3, 1, "f32"),         # fp32 row ending in a half group
    (2, 50, 36, 12, 4, 1, "f32"),        # head size 12: the generic layout, half group
    (2, 50, 72, 24, 6, 0, "bf16"),       # head size 24: generic layout, dw by its own kernel
    (2, 100, 384, 24, 4, 1, "f32"),      # ... in fp32: taps per head for y and dx (a multiple of 8)
    (1, 130, 960, 40, 8, 0, "bf16"),     # head size 40 (5 groups per head), 8 taps
    (2, 40, 2400, 24, 4, 1, "bf16"),     # 100 heads of 24: dw over two blocks of 64 heads, the second partial
    (1, 30, 8400, 120, 3, 0, "bf16"),    # head size 120: dw blocks of 15 x 64 threads
    (2, 70, 1440, 12, 4, 1, "bf16"),     # 120 heads of 12: dw from 4-channel groups, two blocks of 64 heads
    (1, 33, 1400, 20, 5, 0, "f32"),      # 70 heads of 20 in fp32 (16-byte groups of 4), 5 taps
    (2, 20, 960, 60, 3, 1, "bf16"),      # head size 60: dw blocks of 15 x 64 threads, groups of 4
    (1, 25, 680, 68, 4, 1, "bf16"),      # head size 68, past the 4-channel groups: one thread per head
    (1, 5, 16, 8, 8, 1, "bf16"),         # T < W
    (1, 1, 8, 8, 4, 1, "bf16"),          # T = 1
    (4, 97, 16, 16, 7, 1, "f32"),        # 2 lanes per head in fp32, 7 taps
    (1, 1000, 8, 8, 1, 0, "bf16"),       # W = 1
    (2, 150, 1088, 1, 4, 0, "bf16"),     # one channel per filter, taps through LDS: 136 groups, a wave 8/64 full
    (1, 37, 512, 1, 4, 1, "bf16"),       # the same with exactly one wave of 64 groups, T not a multiple of the run
    (2, 40, 256, 1, 4, 1, "bf16"),       # one channel per filter below a wave of groups: the plain layout
]


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dt = str(rng.choice(["f32", "bf16"]))
        Hc = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 3, 6, 12, 40]))
        step = 8 if dt == "bf16" else 4
        m = int(np.lcm(Hc, step))
        D = m * int(rng.integers(1, max(2, 1200 // m)))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 200)), D, Hc, int(rng.integers(1, 9)),
                    int(rng.integers(0, 2)), dt))
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(30, 77), ids=lambda c: "B{}T{}D{}Hc{}W{}r{}{}".format(*c))
def test_headwise_parity_small(case):
    B, T, D, Hc, W, res, dt = case
    wl, seed = headwise_case(B, T, D, Hc, W, res, dt, seed=zlib.crc32(repr(case).encode()))
    inp = draw(wl, seed=seed, need_dy=True)
    x, w, dy = dev(inp["x"]), dev(inp["w"]), dev(inp["dy"])
    y = gpu_fwd(x, w, res)
    dx, dw = gpu_bwd(x, w, dy, res)
    tol = TOL[dt]
    assert_close(host(y), oracle.fwd(inp["x"], inp["w"], res), tol, "y")
    dx_ref, dw_ref = oracle.bwd(inp["x"], inp["w"], inp["dy"], res)
    assert_close(host(dx), dx_ref, tol, "dx")
    assert_close(host(dw), dw_ref, tol, "dw")


def test_tiny_workload_full():
    wl = WORKLOADS["tiny_headwise_f32"]
    inp = draw(wl, need_dy=True)
    x, w = dev(inp["x"]), dev(inp["w"])
    y = gpu_fwd(x, w, wl.residual)
    assert_close(host(y), oracle.fwd(inp["x"], inp["w"], wl.residual), TOL[wl.dtype], "y")


@pytest.mark.parametrize("name", ["qkv_headwise_bf16", "alllinear_headwise_bf16", "mamba2_xbc_headwise_bf16",
                                  "gdn_qkv_headwise_bf16", "qkv_headwise24_bf16"])
def test_full_size_workloads(name):
    """Full sizes, default launch configuration; oracle on sampled tokens."""
    wl = WORKLOADS[name]
    print(f"[{name}] drawing inputs", flush=True)
    inp = draw(wl)
    x, w, dy = dev(inp["x"]), dev(inp["w"]), dev(inp["dy"])
    print(f"[{name}] forward", flush=True)
    y = gpu_fwd(x, w, wl.residual)
    print(f"[{name}] backward", flush=True)
    dx, dw = gpu_bwd(x, w, dy, wl.residual)
    rows = sample_rows(wl.B, wl.T, n_random=40, seed=5)
    tol = TOL[wl.dtype]
    flat = lambda t, n: host(t.reshape(wl.B * wl.T, n)[torch().from_numpy(rows).cuda()])
    print(f"[{name}] oracle on {rows.size} sampled tokens", flush=True)
    assert_close(flat(y, wl.D), oracle.fwd(inp["x"], inp["w"], wl.residual, rows=rows), tol, "y")
    dx_ref, dw_ref = oracle.bwd(inp["x"], inp["w"], inp["dy"], wl.residual, rows=rows)
    assert_close(flat(dx, wl.D), dx_ref, tol, "dx")
    assert_close(flat(dw, wl.G * wl.W).reshape(-1, wl.G, wl.W), dw_ref, tol, "dw")
    # every element written (poisoned with NaN before the call)
    for t, n in ((y, "y"), (dx, "dx"), (dw, "dw")):
        assert bool(torch().isfinite(t).all()), f"{n}: unwritten elements"
    # bit-for-bit repeatable
    y2 = gpu_fwd(x, w, wl.residual)
    dx2, dw2 = gpu_bwd(x, w, dy, wl.residual)
    assert torch().equal(y, y2) and torch().equal(dx, dx2) and torch().equal(dw, dw2)


def test_causality_on_device():
    """Perturbing x[b,s] leaves every y[b,t<s] and every other sequence bitwise unchanged."""
    wl, seed = headwise_case(2, 300, 1024, 8, 4, 1, "bf16", seed=9)
    inp = draw(wl, seed=seed, need_dy=False)
    x, w = dev(inp["x"]), dev(inp["w"])
    y = gpu_fwd(x, w, 1)
    s = 131
    x2 = x.clone()
    x2[1, s] += 1.0
    y2 = gpu_fwd(x2, w, 1)
    assert torch().equal(y2[0], y[0])
    assert torch().equal(y2[1, :s], y[1, :s])
    assert torch().equal(y2[1, s + 4:], y[1, s + 4:])
    assert not torch().equal(y2[1, s], y[1, s])


def test_identity_bitwise():
    """W = 1 with unit filters returns x exactly (residual off) and 2x (residual on)."""
    t = torch()
    x = t.randn(2, 77, 520, device="cuda").to(t.bfloat16)
    w = t.ones(2, 77, 65, 1, device="cuda", dtype=t.bfloat16)
    assert t.equal(gpu_fwd(x, w, 0), x)
    assert t.equal(gpu_fwd(x, w, 1), 2 * x)
