"""Parity of the decode-step HIP kernels (dsc_decode_step, dsc_lowrank_decode_step,
dsc_decode_state_from_prefill) with the CPU oracle.

Replays decode a whole sequence one token at a time from a ring filled with NaN
(slots of steps before 0 must never be read) and compare every step's y with
the oracle and the ring with the oracle's bit for bit. Mixed-position batches
start from prompts of different lengths and include idle rows, which must be
left untouched. The decode workloads at full size are checked on every row.
Tolerance: max |gpu - ref| <= tol * (1 + |ref|), tol 1e-5 (fp32) / 1e-2 (bf16);
ring contents are copies of x and must match exactly.
"""
import zlib

import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
import oracle
from dynamic_short_convolutions_amd.synthetic import (DECODE_WORKLOADS, Workload, draw, draw_decode,
                                                      f32_to_bf16_bits)
from gpu_helpers import TOL, assert_close, check_guard, dev, host, poisoned, torch

pytestmark = pytest.mark.gpu


def bits(t):
    """Raw storage bits of a GPU tensor, as a numpy integer array."""
    tt = torch()
    return t.view(tt.int16 if t.dtype == tt.bfloat16 else tt.int32).cpu().numpy()


def np_bits(a):
    return a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32)


def nan_ring(B, W, D, dt):
    a = np.full((B, W - 1, D), np.nan, np.float32)
    return f32_to_bf16_bits(a) if dt == "bf16" else a


def ipos(v):
    return torch().tensor(np.asarray(v, np.int32), device="cuda")


def run_step(kind, x, f, pos, ring, W, res):
    """One GPU decode step into a poisoned y; f = w (head-wise) or (z, U) (low-rank)."""
    y, ybuf = poisoned(tuple(x.shape), x.dtype)
    if kind == "headwise":
        dsc.dsc_decode_step(x, f, pos, ring, y, res)
    else:
        dsc.dsc_lowrank_decode_step(x, f[0], f[1], pos, ring, y, W, res)
    torch().cuda.synchronize()
    check_guard(ybuf, y.numel(), "y")
    return y


# (kind, B, T, D, Hc or R, W, residual, dtype): every tap count, both dtypes, both
# low-rank paths (matrix cores: bf16 with R a multiple of 8; vector ALU otherwise),
# row counts that leave a ragged block of 16 rows, channel counts that leave a
# ragged channel block, head layouts inside and across 16-byte vectors.
REPLAY_CASES = [
    ("headwise", 3, 12, 64, 8, 4, 1, "bf16"),
    ("headwise", 5, 10, 48, 2, 3, 0, "f32"),
    ("headwise", 2, 9, 72, 24, 6, 1, "bf16"),     # head of 24: 3 vectors per head
    ("headwise", 4, 11, 40, 4, 8, 1, "f32"),
    ("headwise", 3, 6, 16, 1, 1, 1, "bf16"),      # W = 1: no ring
    ("headwise", 17, 7, 96, 12, 2, 0, "bf16"),    # head of 12 straddles vectors
    ("lowrank", 19, 10, 72, 32, 4, 0, "bf16"),    # matrix cores, ragged rows and channels
    ("lowrank", 3, 12, 128, 64, 8, 1, "bf16"),    # matrix cores, two K steps
    ("lowrank", 33, 6, 64, 8, 5, 0, "bf16"),      # three blocks of 16 rows
    ("lowrank", 2, 7, 256, 128, 3, 1, "bf16"),    # the largest rank
    ("lowrank", 4, 9, 64, 16, 1, 1, "bf16"),      # W = 1 on the matrix cores
    ("lowrank", 3, 10, 40, 5, 4, 1, "bf16"),      # R not a multiple of 8: vector ALU
    ("lowrank", 4, 8, 36, 6, 7, 0, "f32"),        # fp32: vector ALU
    ("lowrank", 2, 5, 32, 3, 2, 1, "f32"),
]


def _draw_sequence(kind, B, T, D, HR, W, res, dt):
    seed = zlib.crc32(repr((kind, B, T, D, HR, W, res, dt)).encode())
    if kind == "headwise":
        wl = Workload("dec_hw", kind, B=B, T=T, D=D, W=W, residual=res, dtype=dt, Hc=HR)
    else:
        wl = Workload("dec_lr", kind, B=B, T=T, D=D, W=W, residual=res, dtype=dt, R=HR,
                      U_std=1.0 / np.sqrt(HR * W))
    return draw(wl, seed=seed, need_dy=False)


@pytest.mark.parametrize("case", REPLAY_CASES, ids=lambda c: "{}_B{}T{}D{}_{}W{}r{}{}".format(*c))
def test_decode_replay_matches_oracle(case):
    kind, B, T, D, HR, W, res, dt = case
    inp = _draw_sequence(*case)
    x_all = inp["x"]
    ring_np = nan_ring(B, W, D, dt)
    ring = dev(ring_np) if W > 1 else None
    U = dev(inp["U"]) if kind == "lowrank" else None
    for t in range(T):
        xt = np.ascontiguousarray(x_all[:, t])
        pos_np = np.full(B, t, np.int32)
        if kind == "headwise":
            wt = np.ascontiguousarray(inp["w"][:, t])
            y = run_step(kind, dev(xt), dev(wt), ipos(pos_np), ring, W, res)
            y_ref, ring_np = oracle.decode_step(xt, wt, pos_np, ring_np, res)
        else:
            zt = np.ascontiguousarray(inp["z"][:, t])
            y = run_step(kind, dev(xt), (dev(zt), U), ipos(pos_np), ring, W, res)
            y_ref, ring_np = oracle.lowrank_decode_step(xt, zt, inp["U"], pos_np, ring_np, W, res)
        assert_close(host(y), y_ref, TOL[dt], f"y at step {t}")
        if W > 1:
            assert np.array_equal(bits(ring), np_bits(ring_np)), f"ring after step {t}"
    # and the whole run equals the forward pass over the sequence
    if kind == "headwise":
        y_fwd = oracle.fwd(x_all, inp["w"], res)
    else:
        y_fwd = oracle.lowrank_fwd(x_all, inp["z"], inp["U"], W, res)
    assert_close(host(y), y_fwd[:, T - 1], TOL[dt], "last step vs forward")


@pytest.mark.parametrize("kind,D,HR,W,dt", [("headwise", 64, 8, 4, "bf16"), ("headwise", 32, 4, 7, "f32"),
                                            ("lowrank", 72, 32, 4, "bf16"), ("lowrank", 64, 64, 8, "bf16"),
                                            ("lowrank", 24, 4, 3, "f32")])
def test_prompts_of_mixed_length_and_idle_rows(kind, D, HR, W, dt):
    """Rings filled from prompts of lengths 0 .. T (and past T: clamped), then one step
    at each row's own position; rows with a negative position are idle."""
    T = 20
    lens = np.array([0, 1, W - 2, W - 1, W, 9, T - 1, T, T + 5, 3, 0, 17, 2, 6, 11, 4, 13, 8], np.int32)
    lens = np.maximum(lens, 0)
    B = lens.size
    inp = _draw_sequence(kind, B, T + 1, D, HR, W, 1, dt)
    x_all = inp["x"]
    prompts = np.ascontiguousarray(x_all[:, :T])
    ring0 = nan_ring(B, W, D, dt)
    ring = dev(ring0)
    dsc.dsc_decode_state_from_prefill(dev(prompts), ipos(lens), ring, W)
    torch().cuda.synchronize()
    ring_ref = oracle.decode_state_from_prefill(prompts, lens, ring0)
    assert np.array_equal(bits(ring), np_bits(ring_ref)), "ring after the prompts"

    pos = np.minimum(lens, T).astype(np.int32)
    idle = np.array([3, 10, 15])
    pos[idle] = -1
    rows = np.arange(B)
    t_row = np.maximum(pos, 0)
    xt = np.ascontiguousarray(x_all[rows, t_row])
    if kind == "headwise":
        wt = np.ascontiguousarray(inp["w"][rows, t_row])
        y = run_step(kind, dev(xt), dev(wt), ipos(pos), ring, W, 1)
        y_ref, ring_ref = oracle.decode_step(xt, wt, pos, ring_ref, 1)
        y_fwd = oracle.fwd(x_all, inp["w"], 1)
    else:
        zt = np.ascontiguousarray(inp["z"][rows, t_row])
        y = run_step(kind, dev(xt), (dev(zt), dev(inp["U"])), ipos(pos), ring, W, 1)
        y_ref, ring_ref = oracle.lowrank_decode_step(xt, zt, inp["U"], pos, ring_ref, W, 1)
        y_fwd = oracle.lowrank_fwd(x_all, inp["z"], inp["U"], W, 1)
    active = pos >= 0
    y_h = host(y)
    assert_close(y_h[active], y_ref[active], TOL[dt], "y of active rows")
    assert_close(y_h[active], y_fwd[rows[active], pos[active]], TOL[dt], "y vs the forward pass")
    assert np.isnan(y_h[~active]).all(), "idle rows must leave y untouched"
    assert np.array_equal(bits(ring), np_bits(ring_ref)), "ring after the step"


@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_workloads_full_size(name):
    """The benchmark's decode shapes, every row, plus bit-for-bit repeatability."""
    wl = DECODE_WORKLOADS[name]
    inp = draw_decode(wl)
    # a mix of positions: first tokens, partial rings, full rings, idle rows
    pos = inp["pos"].copy()
    pos[:8] = np.arange(8) % wl.W
    pos[8:12] = -1
    x, ring0 = dev(inp["x"]), dev(inp["state"])
    if wl.kind == "headwise":
        f = dev(inp["w"])
        y_ref, ring_ref = oracle.decode_step(inp["x"], inp["w"], pos, inp["state"], wl.residual)
    else:
        f = (dev(inp["z"]), dev(inp["U"]))
        y_ref, ring_ref = oracle.lowrank_decode_step(inp["x"], inp["z"], inp["U"], pos, inp["state"], wl.W,
                                                     wl.residual)
    print(f"[{name}] GPU step", flush=True)
    ring = ring0.clone()
    y = run_step(wl.kind, x, f, ipos(pos), ring, wl.W, wl.residual)
    active = pos >= 0
    y_h = host(y)
    assert_close(y_h[active], y_ref[active], TOL[wl.dtype], "y")
    assert np.isnan(y_h[~active]).all()
    assert np.array_equal(bits(ring), np_bits(ring_ref)), "ring"
    ring2 = ring0.clone()
    y2 = run_step(wl.kind, x, f, ipos(pos), ring2, wl.W, wl.residual)
    assert np.array_equal(bits(y2)[active], bits(y)[active]) and torch().equal(ring2, ring)


def test_decode_equals_gpu_forward_after_prefill():
    """Prefill with dsc_fwd + ring from the prompt + decode steps reproduces dsc_fwd over
    the whole sequence (head-wise, bf16), within the tolerance."""
    t = torch()
    B, T0, n, D, Hc, W = 4, 37, 6, 512, 8, 4
    inp = _draw_sequence("headwise", B, T0 + n, D, Hc, W, 1, "bf16")
    x, w = dev(inp["x"]), dev(inp["w"])
    y_full = t.empty_like(x)
    dsc.dsc_fwd(x, w, y_full, True)
    ring = t.full((B, W - 1, D), float("nan"), dtype=t.bfloat16, device="cuda")
    dsc.dsc_decode_state_from_prefill(x[:, :T0].contiguous(), ipos(np.full(B, T0)), ring, W)
    for s in range(T0, T0 + n):
        y = run_step("headwise", x[:, s].contiguous(), w[:, s].contiguous(), ipos(np.full(B, s)), ring, W, 1)
        assert_close(host(y), host(y_full[:, s]), TOL["bf16"], f"step {s}")
