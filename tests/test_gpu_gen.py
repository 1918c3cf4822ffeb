"""Parity of the forward with filters generated in the kernel (dsc_fwd_gen) and of its
backward (dsc_bwd_gen: dx and the filters' gradient dw) with the CPU oracle (filters
h . Wg^T in float64, then the forward or the backward). Small shapes on every
element; the QKV layer with a 2048-wide hidden state at full size on sampled
tokens, and against the unfused path (torch's GEMM writing bf16 filters, then
dsc_fwd or dsc_bwd). Tolerance: max |gpu - ref| <= 1e-2 * (1 + |ref|) (bf16).
"""
import zlib

import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
import oracle
from dynamic_short_convolutions_amd.synthetic import WORKLOADS, Workload, draw_gen, packed_positions
from gpu_helpers import TOL, assert_close, check_guard, dev, host, poisoned, sample_rows, torch

pytestmark = pytest.mark.gpu

# (B, T, D, Hc, W, K, residual): G = D / Hc, a multiple of 32
CASES = [
    (2, 300, 256, 8, 4, 128, 1),     # one head block, ragged last step tile
    (1, 130, 512, 16, 3, 64, 0),     # 16 channels per head, one K stage
    (2, 200, 1024, 8, 8, 256, 1),    # four head blocks, 8 taps
    (3, 50, 256, 8, 1, 64, 1),       # W = 1
    (1, 257, 2048, 64, 2, 192, 0),   # 64 channels per head: 256 channel groups per block
    (2, 129, 512, 8, 5, 128, 1),     # two head blocks, 5 taps
    (1, 1, 256, 8, 6, 64, 1),        # T = 1
    (2, 600, 768, 24, 7, 320, 0),    # 24 channels per head, 7 taps, five K stages
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}D{}Hc{}W{}K{}r{}".format(*c))
def test_gen_parity_small(case):
    B, T, D, Hc, W, K, res = case
    wl = Workload("gen", "headwise", B=B, T=T, D=D, W=W, residual=res, dtype="bf16", Hc=Hc)
    inp = draw_gen(wl, K, seed=zlib.crc32(repr(case).encode()))
    x, h, Wg = dev(inp["x"]), dev(inp["h"]), dev(inp["Wg"])
    y, yb = poisoned((B, T, D), x.dtype)
    dsc.dsc_fwd_gen(x, h, Wg, y, W, res)
    torch().cuda.synchronize()
    check_guard(yb, y.numel(), "y")
    assert_close(host(y), oracle.fwd_gen(inp["x"], inp["h"], inp["Wg"], D // Hc, W, res), TOL["bf16"], "y")


def test_gen_workload_full_size():
    t = torch()
    wl = WORKLOADS["qkv_headwise_bf16"]
    K = 2048
    print("[gen] drawing inputs", flush=True)
    inp = draw_gen(wl, K)
    x, h, Wg = dev(inp["x"]), dev(inp["h"]), dev(inp["Wg"])
    y, yb = poisoned((wl.B, wl.T, wl.D), x.dtype)
    print("[gen] GPU", flush=True)
    dsc.dsc_fwd_gen(x, h, Wg, y, wl.W, wl.residual)
    t.cuda.synchronize()
    check_guard(yb, y.numel(), "y")
    rows = sample_rows(wl.B, wl.T, n_random=24, seed=11)
    sel = t.from_numpy(rows).cuda()
    flat = host(y.reshape(-1, wl.D)[sel])
    print(f"[gen] oracle on {rows.size} tokens", flush=True)
    ref = oracle.fwd_gen(inp["x"], inp["h"], inp["Wg"], wl.G, wl.W, wl.residual, rows=rows)
    assert_close(flat, ref, TOL["bf16"], "y")
    # the unfused path (bf16 filters written by torch's GEMM, then the plain forward) is
    # no closer to the oracle: the fused kernel keeps the filters in fp32
    w = t.matmul(h.reshape(-1, K), Wg.t().contiguous()).reshape(wl.B, wl.T, wl.G, wl.W).contiguous()
    y2 = t.empty_like(x)
    dsc.dsc_fwd(x, w, y2, wl.residual)
    t.cuda.synchronize()
    err_fused = np.abs(flat - ref).max()
    err_unfused = np.abs(host(y2.reshape(-1, wl.D)[sel]) - ref).max()
    print(f"[gen] max error fused {err_fused:.3g}, unfused {err_unfused:.3g}", flush=True)
    assert err_fused <= err_unfused
    y3 = t.empty_like(x)
    dsc.dsc_fwd_gen(x, h, Wg, y3, wl.W, wl.residual)
    assert t.equal(y.view(t.int16), y3.view(t.int16))


# ------------------------------------------------------------------ packed sequences

# (B, T, D, Hc, W, K, residual, mean sequence length)
PACKED = [
    (2, 300, 256, 8, 4, 128, 1, 20),     # 256-step tiles, sequences of ~20
    (2, 200, 1024, 8, 8, 64, 0, 6),      # 8 taps, many short sequences
    (1, 257, 512, 16, 3, 192, 1, 3),     # sequences of 1-3 tokens
    (3, 130, 768, 24, 6, 64, 1, 40),
    (2, 90, 256, 8, 1, 64, 0, 5),        # W = 1: positions change nothing
]


def _packed_inputs(case):
    B, T, D, Hc, W, K, res, mean = case
    wl = Workload("genp", "headwise", B=B, T=T, D=D, W=W, residual=res, dtype="bf16", Hc=Hc)
    seed = zlib.crc32(repr(case).encode())
    inp = draw_gen(wl, K, seed=seed)
    inp["pos"] = packed_positions(B, T, mean, seed + 5)
    return inp


def _run_packed(x, h, Wg, pos, W, res):
    t = torch()
    y, yb = poisoned(tuple(x.shape), x.dtype)
    dsc.dsc_fwd_gen_varlen(x, h, Wg, t.from_numpy(pos).cuda(), y, W, res)
    t.cuda.synchronize()
    check_guard(yb, y.numel(), "y")
    return y


@pytest.mark.parametrize("case", PACKED, ids=lambda c: "B{}T{}D{}Hc{}W{}K{}r{}_L{}".format(*c))
def test_gen_packed_parity(case):
    B, T, D, Hc, W, K, res, mean = case
    inp = _packed_inputs(case)
    y = _run_packed(dev(inp["x"]), dev(inp["h"]), dev(inp["Wg"]), inp["pos"], W, res)
    ref = oracle.fwd_gen(inp["x"], inp["h"], inp["Wg"], D // Hc, W, res, pos=inp["pos"])
    assert_close(host(y), ref, TOL["bf16"], "y")


def test_gen_positions_from_zero_equal_dense_bitwise():
    """pos[t] = t is the dense operation: the packed call gives dsc_fwd_gen's bits."""
    t = torch()
    B, T, D, Hc, W, K, res, _ = PACKED[0]
    inp = _packed_inputs(PACKED[0])
    x, h, Wg = dev(inp["x"]), dev(inp["h"]), dev(inp["Wg"])
    pos = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    y = _run_packed(x, h, Wg, pos, W, res)
    y0 = t.empty_like(x)
    dsc.dsc_fwd_gen(x, h, Wg, y0, W, res)
    t.cuda.synchronize()
    assert t.equal(y.view(t.int16), y0.view(t.int16))


def test_gen_nan_stays_in_its_sequence():
    """A NaN in one sequence's x changes no output of any other sequence."""
    t = torch()
    case = PACKED[0]
    B, T, D, Hc, W, K, res, _ = case
    inp = _packed_inputs(case)
    pos = inp["pos"]
    starts = np.flatnonzero(pos[0] == 0)
    s0, s1 = int(starts[2]), int(starts[3])  # the third sequence of row 0
    x2 = inp["x"].copy()
    x2[0, s0:s1, :5] = 0x7FC0  # bf16 NaN
    other = np.ones((B, T), bool)
    other[0, s0:s1] = False
    h, Wg = dev(inp["h"]), dev(inp["Wg"])
    a = _run_packed(dev(inp["x"]), h, Wg, pos, W, res)
    b = _run_packed(dev(x2), h, Wg, pos, W, res)
    m = t.from_numpy(other).cuda()
    assert t.equal(a[m].view(t.int16), b[m].view(t.int16))
    assert bool(t.isnan(b[0, s0:s1].float()).any())


# ------------------------------------------------------------------ backward

# (B, T, D, Hc, W, K, residual): backward step tiles are 125 steps (W <= 4, 128 - 3)
# or 64 - W + 1 (W > 4); D/Hc/8 a power of two
BWD_CASES = [
    (2, 300, 256, 8, 4, 128, 1),     # one head block, tiles of 125: ragged last tile
    (1, 250, 512, 16, 3, 64, 0),     # tile edge at 126, head sums over 2 lanes
    (2, 200, 1024, 8, 8, 256, 1),    # four head blocks, 8 taps, tiles of 57
    (3, 50, 256, 8, 1, 64, 1),       # W = 1: no filter rows from the next tile
    (1, 257, 2048, 64, 2, 192, 0),   # 64 channels per head: sums over 8 lanes
    (1, 131, 4096, 128, 5, 64, 1),   # 128 channels per head: sums over 16 lanes
    (2, 129, 512, 8, 5, 128, 1),     # two head blocks, 5 taps
    (1, 1, 256, 8, 6, 64, 1),        # T = 1
    (1, 3, 1024, 32, 7, 64, 0),      # T < W
    (2, 600, 1024, 32, 7, 320, 0),   # 7 taps, five K stages, 4-lane head sums
]


def _with_dy(inp, seed):
    """dy ~ N(0, 1) as bf16 bit patterns (truncated float32), beside draw_gen's inputs."""
    rng = np.random.default_rng(seed)
    inp["dy"] = (rng.standard_normal(inp["x"].shape, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return inp


def _bwd_inputs(case):
    B, T, D, Hc, W, K, res = case[:7]
    wl = Workload("genb", "headwise", B=B, T=T, D=D, W=W, residual=res, dtype="bf16", Hc=Hc)
    seed = zlib.crc32(repr(case).encode())
    return wl, _with_dy(draw_gen(wl, K, seed=seed), seed + 1)


def _run_bwd(inp, G, W, res, pos=None):
    t = torch()
    x, h, Wg, dy = dev(inp["x"]), dev(inp["h"]), dev(inp["Wg"]), dev(inp["dy"])
    B, T, D = x.shape
    dx, dxb = poisoned((B, T, D), x.dtype)
    dw, dwb = poisoned((B, T, G, W), x.dtype)
    if pos is None:
        dsc.dsc_bwd_gen(x, h, Wg, dy, dx, dw, W, res)
    else:
        dsc.dsc_bwd_gen_varlen(x, h, Wg, t.from_numpy(pos).cuda(), dy, dx, dw, W, res)
    t.cuda.synchronize()
    check_guard(dxb, dx.numel(), "dx")
    check_guard(dwb, dw.numel(), "dw")
    return dx, dw


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}T{}D{}Hc{}W{}K{}r{}".format(*c))
def test_gen_bwd_parity_small(case):
    B, T, D, Hc, W, K, res = case
    wl, inp = _bwd_inputs(case)
    dx, dw = _run_bwd(inp, wl.G, W, res)
    dx_r, dw_r = oracle.bwd_gen(inp["x"], inp["h"], inp["Wg"], inp["dy"], wl.G, W, res)
    assert_close(host(dx), dx_r, TOL["bf16"], "dx")
    assert_close(host(dw), dw_r, TOL["bf16"], "dw")


def test_gen_bwd_unsupported_head_width():
    """24 channels per head (3 groups of 8) has a forward but no fused backward."""
    wl, inp = _bwd_inputs((1, 8, 768, 24, 4, 64, 1))
    with pytest.raises(dsc.DscError, match="NOT_SUPPORTED"):
        _run_bwd(inp, wl.G, 4, 1)


# (B, T, D, Hc, W, K, residual, mean sequence length)
BWD_PACKED = [
    (2, 300, 256, 8, 4, 128, 1, 20),
    (2, 200, 1024, 8, 8, 64, 0, 6),
    (1, 257, 512, 16, 3, 192, 1, 3),
    (3, 130, 1024, 32, 6, 64, 1, 40),
    (2, 90, 256, 8, 1, 64, 0, 5),
]


@pytest.mark.parametrize("case", BWD_PACKED, ids=lambda c: "B{}T{}D{}Hc{}W{}K{}r{}_L{}".format(*c))
def test_gen_bwd_packed_parity(case):
    B, T, D, Hc, W, K, res, mean = case
    wl, inp = _bwd_inputs(case)
    pos = packed_positions(B, T, mean, zlib.crc32(repr(case).encode()) + 5)
    dx, dw = _run_bwd(inp, wl.G, W, res, pos=pos)
    dx_r, dw_r = oracle.bwd_gen(inp["x"], inp["h"], inp["Wg"], inp["dy"], wl.G, W, res, pos=pos)
    assert_close(host(dx), dx_r, TOL["bf16"], "dx")
    assert_close(host(dw), dw_r, TOL["bf16"], "dw")


def test_gen_bwd_positions_from_zero_equal_dense_bitwise():
    t = torch()
    case = BWD_PACKED[0]
    B, T, D, Hc, W, K, res, _ = case
    wl, inp = _bwd_inputs(case)
    pos = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    dx, dw = _run_bwd(inp, wl.G, W, res, pos=pos)
    dx0, dw0 = _run_bwd(inp, wl.G, W, res)
    assert t.equal(dx.view(t.int16), dx0.view(t.int16)) and t.equal(dw.view(t.int16), dw0.view(t.int16))


def test_gen_bwd_workload_full_size():
    """The QKV layer (2048-wide hidden state) at full size: sampled tokens against the
    oracle, the unfused path (torch's GEMM writing bf16 filters, then dsc_bwd): its dw
    is the same function of x and dy (bitwise: the filters do not enter it), and a
    second call gives the same bits."""
    t = torch()
    wl = WORKLOADS["qkv_headwise_bf16"]
    K = 2048
    print("[gen bwd] drawing inputs", flush=True)
    inp = _with_dy(draw_gen(wl, K), 20261215)
    print("[gen bwd] GPU", flush=True)
    dx, dw = _run_bwd(inp, wl.G, wl.W, wl.residual)
    rows = sample_rows(wl.B, wl.T, n_random=24, seed=12)
    # tile edges of the backward (125-step tiles) and of the forward (256)
    edges = np.array([124, 125, 126, 249, 250, 255, 256, 3999, 4000, 4001], dtype=np.int64)
    rows = np.unique(np.concatenate([rows, edges[edges < wl.T], (wl.B - 1) * wl.T + edges[edges < wl.T]]))
    sel = t.from_numpy(rows).cuda()
    print(f"[gen bwd] oracle on {rows.size} tokens", flush=True)
    dx_r, dw_r = oracle.bwd_gen(inp["x"], inp["h"], inp["Wg"], inp["dy"], wl.G, wl.W, wl.residual, rows=rows)
    assert_close(host(dx.reshape(-1, wl.D)[sel]), dx_r, TOL["bf16"], "dx")
    assert_close(host(dw.reshape(-1, wl.G, wl.W)[sel]), dw_r, TOL["bf16"], "dw")
    x, h, Wg, dy = dev(inp["x"]), dev(inp["h"]), dev(inp["Wg"]), dev(inp["dy"])
    w = t.matmul(h.reshape(-1, K), Wg.t().contiguous()).reshape(wl.B, wl.T, wl.G, wl.W).contiguous()
    dx2, dw2 = t.empty_like(x), t.empty_like(w)
    dsc.dsc_bwd(x, w, dy, dx2, dw2, wl.residual)
    t.cuda.synchronize()
    err_fused = np.abs(host(dx.reshape(-1, wl.D)[sel]) - dx_r).max()
    err_unfused = np.abs(host(dx2.reshape(-1, wl.D)[sel]) - dx_r).max()
    print(f"[gen bwd] dx max error fused {err_fused:.3g}, unfused {err_unfused:.3g}", flush=True)
    assert err_fused <= err_unfused
    dx3, dw3 = _run_bwd(inp, wl.G, wl.W, wl.residual)
    assert t.equal(dx.view(t.int16), dx3.view(t.int16)) and t.equal(dw.view(t.int16), dw3.view(t.int16))
