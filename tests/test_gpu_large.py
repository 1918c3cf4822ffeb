"""Tensors past 2^31 elements: the head-wise and low-rank passes on a batch of 65
sequences of 8192 steps by 4096 channels (2.18e9 elements, 4.4 GB per bf16
activation), so the last sequence starts 2^31 elements (4 GiB) into each tensor.

The first and the last sequence are drawn by the shared input generator and their
outputs are checked against the oracle on sampled steps (sequence starts and ends,
tile edges, random steps); the sequences between are filled on the device (each
sequence is computed on its own, so their values only have to be finite), and every
output element must be written. dU, a sum over every sequence, is checked on the
columns of a few channels: a column of channel c only involves channel c of x and
dy (and all of z), so those channels of every sequence are gathered on the device,
copied back, and the oracle's per-sequence sums are added in double on the host.
Tolerance: max |gpu - ref| <= 1e-2 * (1 + |ref|) (bf16).
"""
import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
import oracle
from dynamic_short_convolutions_amd.synthetic import Workload, draw
from gpu_helpers import TOL, assert_close, dev, host, sample_rows, torch

pytestmark = pytest.mark.gpu

B, T, D = 65, 8192, 4096


def _device_fill(shape, seed):
    """bf16 N(0, 1) values, one sequence at a time (keeps the fp32 temporaries small)."""
    t = torch()
    out = t.empty(shape, dtype=t.bfloat16, device="cuda")
    g = t.Generator(device="cuda")
    g.manual_seed(seed)
    for b in range(shape[0]):
        out[b] = t.randn(shape[1:], device="cuda", generator=g, dtype=t.float32).to(t.bfloat16)
    return out


def _place(big, name, first, last):
    big[0].copy_(dev(first[name][0]))
    big[B - 1].copy_(dev(last[name][0]))


def _check_rows(gpu, ref_fn, rows, what):
    """gpu: [T, C] tensor of one sequence; ref_fn(rows) -> oracle rows."""
    idx = torch().from_numpy(rows).cuda()
    assert_close(host(gpu[idx]), ref_fn(rows), TOL["bf16"], what)


def test_headwise_past_2_31_elements():
    t = torch()
    assert B * T * D > 2 ** 31 and (B - 1) * T * D >= 2 ** 31
    wl = Workload("large_hw", "headwise", B=1, T=T, D=D, W=4, residual=1, dtype="bf16", Hc=8)
    first, last = draw(wl, seed=20261311, need_dy=True), draw(wl, seed=20261312, need_dy=True)
    print("[large head-wise] filling the batch", flush=True)
    x = _device_fill((B, T, D), 1)
    w = _device_fill((B, T, wl.G, wl.W), 2)
    dy = _device_fill((B, T, D), 3)
    for big, name in ((x, "x"), (w, "w"), (dy, "dy")):
        _place(big, name, first, last)
    y = t.full_like(x, float("nan"))
    dx = t.full_like(x, float("nan"))
    dw = t.full_like(w, float("nan"))
    print("[large head-wise] forward and backward", flush=True)
    dsc.dsc_fwd(x, w, y, True)
    dsc.dsc_bwd(x, w, dy, dx, dw, True)
    t.cuda.synchronize()
    for o, n in ((y, "y"), (dx, "dx"), (dw, "dw")):
        assert bool(t.isfinite(o).all()), f"{n}: unwritten elements"
    rows = sample_rows(1, T, n_random=32, seed=12)
    for b, inp in ((0, first), (B - 1, last)):
        print(f"[large head-wise] oracle, sequence {b}", flush=True)
        _check_rows(y[b], lambda r: oracle.fwd(inp["x"], inp["w"], 1, rows=r), rows, f"y[{b}]")
        dx_r, dw_r = oracle.bwd(inp["x"], inp["w"], inp["dy"], 1, rows=rows)
        _check_rows(dx[b], lambda r: dx_r, rows, f"dx[{b}]")
        _check_rows(dw[b].reshape(T, -1), lambda r: dw_r.reshape(r.size, -1), rows, f"dw[{b}]")
    del x, w, dy, y, dx, dw
    t.cuda.empty_cache()


def test_lowrank_past_2_31_elements():
    t = torch()
    R, W = 32, 4
    wl = Workload("large_lr", "lowrank", B=1, T=T, D=D, W=W, residual=0, dtype="bf16", R=R,
                  U_std=1.0 / np.sqrt(R * W))
    first, last = draw(wl, seed=20261313, need_dy=True), draw(wl, seed=20261314, need_dy=True)
    last["U"] = first["U"]  # one U for the batch
    print("[large low-rank] filling the batch", flush=True)
    x = _device_fill((B, T, D), 4)
    z = _device_fill((B, T, R), 5)
    dy = _device_fill((B, T, D), 6)
    for big, name in ((x, "x"), (z, "z"), (dy, "dy")):
        _place(big, name, first, last)
    U = dev(first["U"])
    y = t.full_like(x, float("nan"))
    dx = t.full_like(x, float("nan"))
    dz = t.full_like(z, float("nan"))
    dU = t.full_like(U, float("nan"))
    n = dsc.dsc_lowrank_bwd_workspace_bytes(B, T, D, R, W, dsc.DSC_BF16)
    ws = t.empty(max(n, 16), dtype=t.uint8, device="cuda")
    print("[large low-rank] forward and backward", flush=True)
    dsc.dsc_lowrank_fwd(x, z, U, y, W, 0)
    dsc.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, ws, W, 0)
    t.cuda.synchronize()
    for o, nm in ((y, "y"), (dx, "dx"), (dz, "dz"), (dU, "dU")):
        assert bool(t.isfinite(o).all()), f"{nm}: unwritten elements"
    rows = sample_rows(1, T, n_random=32, seed=13)
    for b, inp in ((0, first), (B - 1, last)):
        print(f"[large low-rank] oracle, sequence {b}", flush=True)
        _check_rows(y[b], lambda r: oracle.lowrank_fwd(inp["x"], inp["z"], inp["U"], W, 0, rows=r), rows,
                    f"y[{b}]")
        dx_r, dz_r = oracle.lowrank_bwd_rows(inp["x"], inp["z"], inp["U"], inp["dy"], W, 0, rows=rows)
        _check_rows(dx[b], lambda r: dx_r, rows, f"dx[{b}]")
        _check_rows(dz[b], lambda r: dz_r, rows, f"dz[{b}]")
    # dU on the columns of a few channels (first, block edges, last), summed over all 65 sequences
    chans = np.array([0, 1, 15, 16, 127, 128, 2047, 2048, D - 2, D - 1])
    idx = t.from_numpy(chans).cuda()
    as_bits = lambda a: a.contiguous().cpu().view(t.int16).numpy().view(np.uint16)
    ref = np.zeros((R, chans.size * W))
    print("[large low-rank] dU columns over every sequence", flush=True)
    for b in range(B):
        xs, dys = as_bits(x[b][:, idx])[None], as_bits(dy[b][:, idx])[None]
        ref += oracle.lowrank_dU(xs, as_bits(z[b])[None], dys, W)
    cols = t.from_numpy((chans[:, None] * W + np.arange(W)[None, :]).reshape(-1)).cuda()
    assert_close(host(dU[:, cols]), ref, TOL["bf16"], "dU (sampled columns, all sequences)")
    del x, z, dy, y, dx, dz, dU, ws
    t.cuda.empty_cache()


def test_lowrank_dz_partials_past_2_gib():
    """One sequence of 2^24 + 16 steps at R = 32: its fp32 dz partial [T][R] would be
    2^31 + 2 KiB, past what one buffer resource addresses, so the launch plan takes the
    separate dz pass (a fused partial would lose the last 16 steps' dz). Checked on
    windows of steps around the 2^24 boundary and at both ends (each window run through
    the oracle on its own, rows whose taps reach outside it left out), and on sampled
    dU columns over all steps."""
    t = torch()
    Tl, Dl, R, W = 2 ** 24 + 16, 16, 32, 4
    g = t.Generator(device="cuda")
    g.manual_seed(20261320)
    bf = lambda *shape: t.randn(*shape, device="cuda", generator=g, dtype=t.float32).to(t.bfloat16)
    print("[dz partials past 2 GiB] inputs", flush=True)
    x, z, dy = bf(1, Tl, Dl), bf(1, Tl, R), bf(1, Tl, Dl)
    U = (bf(R, Dl * W).float() / np.sqrt(R * W)).to(t.bfloat16)
    dx, dz, dU = (t.full_like(a, float("nan")) for a in (x, z, U))
    y = t.full_like(x, float("nan"))
    n = dsc.dsc_lowrank_bwd_workspace_bytes(1, Tl, Dl, R, W, dsc.DSC_BF16)
    ws = t.empty(max(n, 16), dtype=t.uint8, device="cuda")
    print("[dz partials past 2 GiB] forward and backward", flush=True)
    dsc.dsc_lowrank_fwd(x, z, U, y, W, 0)
    dsc.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, ws, W, 0)
    t.cuda.synchronize()
    for o, nm in ((y, "y"), (dx, "dx"), (dz, "dz"), (dU, "dU")):
        assert bool(t.isfinite(o).all()), f"{nm}: unwritten elements"
    as_bits = lambda a: a.contiguous().cpu().view(t.int16).numpy().view(np.uint16)
    Ub = as_bits(U)
    for c in (0, 7, 2 ** 23, 2 ** 24 - 40, 2 ** 24 - 9, 2 ** 24 + 3, Tl - 10):
        lo, hi = max(0, c - 12), min(Tl, c + 12)
        xw, zw, dyw = (as_bits(a[:, lo:hi]) for a in (x, z, dy))
        y_r = oracle.lowrank_fwd(xw, zw, Ub, W, 0)
        dx_r, dz_r = oracle.lowrank_bwd_rows(xw, zw, Ub, dyw, W, 0)
        past = 0 if lo == 0 else W - 1      # rows whose taps reach before the window
        future = 0 if hi == Tl else W - 1   # rows whose dx needs steps after it
        sl = slice(lo + past, hi - future)
        w_sl = slice(past, hi - lo - future)
        what = f"steps [{sl.start}, {sl.stop})"
        assert_close(host(y[0, sl]), y_r[0, w_sl], TOL["bf16"], f"y {what}")
        assert_close(host(dx[0, sl]), dx_r[0, w_sl], TOL["bf16"], f"dx {what}")
        assert_close(host(dz[0, sl]), dz_r[0, w_sl], TOL["bf16"], f"dz {what}")
    print("[dz partials past 2 GiB] dU columns", flush=True)
    cols = np.array([0, 3, 5, 30, 63])
    ref = oracle.lowrank_dU(as_bits(x), as_bits(z), as_bits(dy), W, cols=cols)
    assert_close(host(dU[:, t.from_numpy(cols).cuda()]), ref, TOL["bf16"], "dU (sampled columns)")
    del x, z, dy, y, dx, dz, dU, ws
    t.cuda.empty_cache()
