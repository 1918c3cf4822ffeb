"""The entry points under HIP graph capture.

They only enqueue kernels on the caller's stream (no allocation, memset or
synchronisation inside), so a captured forward + backward must replay to the same
bits as the eager calls. Between replays the outputs are overwritten by eager work
on the program's own stream and the device is synchronised; every replay is
compared with the eager result.
"""
import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
from dynamic_short_convolutions_amd.synthetic import Workload, draw, draw_gen
from gpu_helpers import dev, torch

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replay_and_compare(run, outputs):
    """run() enqueues the calls on the current stream; outputs are the tensors it writes."""
    t = torch()
    run()
    t.cuda.synchronize()
    eager = [o.clone() for o in outputs]

    g = t.cuda.CUDAGraph()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        run()  # warm-up on the capture stream, outside the graph
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    with t.cuda.graph(g):
        run()
    for rep in range(REPLAYS):
        for o in outputs:
            o.fill_(float("nan"))  # eager work on the same memory between replays
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert t.equal(o.view(t.int16) if o.dtype == t.bfloat16 else o.view(t.int32),
                           e.view(t.int16) if e.dtype == t.bfloat16 else e.view(t.int32)), f"replay {rep}"


def test_headwise_fwd_bwd_graph():
    t = torch()
    wl = Workload("graph_hw", "headwise", B=2, T=150, D=128, W=4, residual=1, dtype="bf16", Hc=8)
    inp = draw(wl, 20261301, True)
    x, w, dy = dev(inp["x"]), dev(inp["w"]), dev(inp["dy"])
    y, dx, dw = t.empty_like(x), t.empty_like(x), t.empty_like(w)

    def run():
        dsc.dsc_fwd(x, w, y, True)
        dsc.dsc_bwd(x, w, dy, dx, dw, True)

    _replay_and_compare(run, [y, dx, dw])


@pytest.mark.parametrize("R,W", [(32, 4), (64, 8)])
def test_lowrank_fwd_bwd_graph(R, W):
    t = torch()
    wl = Workload(f"graph_lr_R{R}", "lowrank", B=2, T=200, D=128, W=W, residual=0, dtype="bf16", R=R,
                  U_std=1.0 / np.sqrt(R * W))
    inp = draw(wl, 20261302, True)
    x, z, U, dy = dev(inp["x"]), dev(inp["z"]), dev(inp["U"]), dev(inp["dy"])
    y, dx, dz, dU = t.empty_like(x), t.empty_like(x), t.empty_like(z), t.empty_like(U)
    n = dsc.dsc_lowrank_bwd_workspace_bytes(wl.B, wl.T, wl.D, R, W, dsc.DSC_BF16)
    ws = t.empty((max(n, 16),), dtype=t.uint8, device="cuda")

    def run():
        dsc.dsc_lowrank_fwd(x, z, U, y, W, False)
        dsc.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, ws, W, False)

    _replay_and_compare(run, [y, dx, dz, dU])


@pytest.mark.parametrize("kind", ["headwise", "lowrank"])
def test_decode_step_graph(kind):
    """A captured decode step replays to the eager bits. The step updates its ring in
    place, so the ring is restored (eagerly) before the eager call and every replay."""
    t = torch()
    rng = np.random.default_rng(20261303)
    B, D, W = 37, 256, 4
    x = t.from_numpy(rng.standard_normal((B, D), dtype=np.float32)).cuda().to(t.bfloat16)
    ring = t.from_numpy(rng.standard_normal((B, W - 1, D), dtype=np.float32)).cuda().to(t.bfloat16)
    pos = t.from_numpy(rng.integers(-1, 12, size=B).astype(np.int32)).cuda()
    y = t.full_like(x, float("nan"))
    if kind == "headwise":
        w = t.from_numpy(rng.standard_normal((B, D // 8, W), dtype=np.float32)).cuda().to(t.bfloat16)
        run = lambda: dsc.dsc_decode_step(x, w, pos, ring, y, True)
    else:
        R = 32
        z = t.from_numpy(rng.standard_normal((B, R), dtype=np.float32)).cuda().to(t.bfloat16)
        U = (t.from_numpy(rng.standard_normal((R, D * W), dtype=np.float32)) / np.sqrt(R * W)).cuda().to(t.bfloat16)
        run = lambda: dsc.dsc_lowrank_decode_step(x, z, U, pos, ring, y, W, False)
    saved = ring.clone()
    run()
    t.cuda.synchronize()
    y_eager, ring_eager = y.clone(), ring.clone()

    g = t.cuda.CUDAGraph()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        run()  # warm-up on the capture stream, outside the graph
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    with t.cuda.graph(g):
        run()
    for rep in range(REPLAYS):
        ring.copy_(saved)
        y.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(y.view(t.int16), y_eager.view(t.int16)), f"y, replay {rep}"
        assert t.equal(ring.view(t.int16), ring_eager.view(t.int16)), f"ring, replay {rep}"


def test_fwd_gen_graph():
    """The forward and backward with filters generated in the kernel: two head blocks,
    two K stages, ragged last step tiles (256 and 125 steps)."""
    t = torch()
    wl = Workload("graph_gen", "headwise", B=2, T=300, D=512, W=4, residual=1, dtype="bf16", Hc=8)
    inp = draw_gen(wl, 128, seed=20261302)
    x, h, Wg = dev(inp["x"]), dev(inp["h"]), dev(inp["Wg"])
    g = t.Generator(device="cuda")
    g.manual_seed(20261303)
    dy = t.randn(x.shape, device="cuda", generator=g, dtype=t.float32).to(t.bfloat16)
    y, dx = t.empty_like(x), t.empty_like(x)
    dw = t.empty((wl.B, wl.T, wl.G, wl.W), dtype=t.bfloat16, device="cuda")

    def run():
        dsc.dsc_fwd_gen(x, h, Wg, y, wl.W, True)
        dsc.dsc_bwd_gen(x, h, Wg, dy, dx, dw, wl.W, True)

    _replay_and_compare(run, [y, dx, dw])
