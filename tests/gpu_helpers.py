"""Helpers for the GPU parity tests: device transfer, tolerance checks, poisoned
outputs with guard bands, and the rows/columns sampled at full size."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 1e-2}   # max |gpu - ref| <= tol * (1 + |ref|), elementwise
GUARD = 4096                          # elements after every output that must stay untouched
SENTINEL = 12288.0                   # exact in bf16 and fp32


def torch():
    import torch as t

    return t


def have_gpu() -> bool:
    try:
        import torch as t

        return t.cuda.is_available()
    except Exception:
        return False


def dev(a: np.ndarray):
    """Storage array (float32, or bf16 bit patterns as uint16) -> GPU tensor of that dtype."""
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(t.bfloat16)
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(x) -> np.ndarray:
    """GPU tensor -> float64 numpy (bf16 widens exactly)."""
    return x.float().cpu().numpy().astype(np.float64)


def poisoned(shape, dtype):
    """An output tensor filled with NaN, followed in memory by GUARD sentinel elements.
    Returns (view, buffer): check_guard(buffer, view.numel()) verifies the band."""
    t = torch()
    n = int(np.prod(shape))
    buf = t.full((n + GUARD,), float("nan"), dtype=dtype, device="cuda")
    buf[n:] = SENTINEL
    return buf[:n].view(*shape), buf


def check_guard(buf, n: int, what: str) -> None:
    tail = buf[n:].float()
    assert bool((tail == SENTINEL).all()), f"{what}: write past the end of the output"


def assert_close(gpu: np.ndarray, ref: np.ndarray, tol: float, what: str) -> None:
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: {np.size(gpu) - np.isfinite(gpu).sum()} unwritten/non-finite elements"
    err = np.abs(gpu - ref)
    bound = tol * (1.0 + np.abs(ref))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        where = np.argwhere(bad)
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} elements out of tolerance; worst at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r} err={err[i]:.3g} bound={bound[i]:.3g}; "
                             f"first bad indices {where[:12].tolist()}")


def sample_rows(B: int, T: int, n_random: int, seed: int, tiles=(16, 32, 64)) -> np.ndarray:
    """Flat token indices b*T+t: sequence starts and ends, tile edges, and random steps."""
    rng = np.random.default_rng(seed)
    ts = {0, 1, 2, 3, 7, T - 1, T - 2, T - 3}
    for L in tiles:
        for m in (1, 2, 3, T // L // 2, T // L - 1):
            for d in (-1, 0, 1):
                ts.add(m * L + d)
    ts = sorted(t for t in ts if 0 <= t < T)
    rows = {b * T + t for b in {0, B - 1, B // 2} for t in ts}
    rows |= set(rng.integers(0, B * T, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)
