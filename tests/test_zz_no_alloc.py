"""dsc_lowrank_bwd_noalloc: the low-rank backward with the library's own scratch array
in place of a caller's workspace, through the C ABI.

Its outputs must equal dsc_lowrank_bwd's (same kernels, same fixed summation order:
bit for bit, which is within the parity tolerance a fortiori) on two calls in a row,
the second with a smaller problem, on every path the backward takes (the fused dz
pass at R <= 32, the separate dz pass at R = 64, W = 8, and the vector-ALU kernels,
which need no scratch); one shape is also checked against the oracle. A problem
whose workspace exceeds the array is refused before anything is enqueued.
"""
import numpy as np
import pytest

import dynamic_short_convolutions_amd as dsc
import oracle
from dynamic_short_convolutions_amd.synthetic import Workload, draw
from gpu_helpers import TOL, assert_close, dev, host, torch

pytestmark = pytest.mark.gpu


def _inputs(B, T, D, R, W, dtype, seed):
    wl = Workload("noalloc", "lowrank", B=B, T=T, D=D, W=W, residual=0, dtype=dtype, R=R,
                  U_std=1.0 / np.sqrt(R * W))
    inp = draw(wl, seed=seed, need_dy=True)
    return inp, {k: dev(v) for k, v in inp.items()}


def _outputs(t):
    th = torch()
    return tuple(th.full_like(t[k], float("nan")) for k in ("x", "z", "U"))


def _with_workspace(t, W, residual):
    th = torch()
    B, T, D = t["x"].shape
    R = t["z"].shape[2]
    code = dsc.DSC_BF16 if t["x"].dtype == th.bfloat16 else dsc.DSC_F32
    n = dsc.dsc_lowrank_bwd_workspace_bytes(B, T, D, R, W, code)
    ws = th.empty(max(n, 16), dtype=th.uint8, device="cuda") if n else None
    dx, dz, dU = _outputs(t)
    dsc.dsc_lowrank_bwd(t["x"], t["z"], t["U"], t["dy"], dx, dz, dU, ws, W, residual)
    return dx, dz, dU, n


def _no_alloc(t, W, residual):
    dx, dz, dU = _outputs(t)
    dsc.dsc_lowrank_bwd_noalloc(t["x"], t["z"], t["U"], t["dy"], dx, dz, dU, W, residual)
    return dx, dz, dU


# (B, T, D, R, W, dtype): first call, then a smaller one
CASES = [
    ((4, 2048, 1024, 32, 4, "bf16"), (2, 700, 256, 32, 4, "bf16")),     # fused dz pass
    ((1, 8192, 1024, 64, 8, "bf16"), (1, 1000, 512, 64, 8, "bf16")),    # separate dz pass
    ((2, 300, 64, 16, 3, "f32"), (1, 50, 16, 12, 2, "f32")),            # vector-ALU kernels, no scratch
]


@pytest.mark.parametrize("first,second", CASES)
def test_no_alloc_equals_workspace_call(first, second):
    th = torch()
    for i, (B, T, D, R, W, dtype) in enumerate((first, second)):
        print(f"[no-alloc] call {i + 1}: B={B} T={T} D={D} R={R} W={W} {dtype}", flush=True)
        inp, t = _inputs(B, T, D, R, W, dtype, seed=700 + 10 * i + R)
        residual = i % 2
        ref = _with_workspace(t, W, residual)
        got = _no_alloc(t, W, residual)
        th.cuda.synchronize()
        assert ref[3] <= dsc.NOALLOC_SCRATCH_BYTES
        for name, a, b in zip(("dx", "dz", "dU"), got, ref[:3]):
            assert bool(th.isfinite(a).all()), f"{name}: unwritten elements"
            assert th.equal(a, b), f"{name} differs from dsc_lowrank_bwd's"


def test_no_alloc_against_the_oracle():
    B, T, D, R, W = 2, 333, 128, 32, 4
    inp, t = _inputs(B, T, D, R, W, "bf16", seed=731)
    dx, dz, dU = _no_alloc(t, W, 1)
    torch().cuda.synchronize()
    dx_r, dz_r, dU_r = oracle.lowrank_bwd(inp["x"], inp["z"], inp["U"], inp["dy"], W, 1)
    assert_close(host(dx), dx_r, TOL["bf16"], "dx")
    assert_close(host(dz), dz_r, TOL["bf16"], "dz")
    assert_close(host(dU), dU_r, TOL["bf16"], "dU")


def test_no_alloc_refuses_a_problem_beyond_its_scratch():
    th = torch()
    B, T, D, R, W = 16, 4096, 2048, 32, 4
    assert dsc.dsc_lowrank_bwd_workspace_bytes(B, T, D, R, W, dsc.DSC_BF16) > dsc.NOALLOC_SCRATCH_BYTES
    x = th.zeros((B, T, D), dtype=th.bfloat16, device="cuda")
    z = th.zeros((B, T, R), dtype=th.bfloat16, device="cuda")
    U = th.zeros((R, D * W), dtype=th.bfloat16, device="cuda")
    dy = th.zeros_like(x)
    dx, dz, dU = th.full_like(x, float("nan")), th.full_like(z, float("nan")), th.full_like(U, float("nan"))
    with pytest.raises(dsc.DscError) as e:
        dsc.dsc_lowrank_bwd_noalloc(x, z, U, dy, dx, dz, dU, W, 0)
    assert e.value.status == 5  # DSC_ERROR_WORKSPACE
    th.cuda.synchronize()
    assert bool(th.isnan(dx).all()) and bool(th.isnan(dU).all()), "nothing may be enqueued"
