"""Pins of the oracle's packed-sequence form (per-token positions) against the
dense oracle, which the other pin files tie to the method's definition.

Several sequences packed into one row, with pos[t] the index of token t within
its own sequence, must give exactly what the dense oracle gives on each
sequence alone ("Dynamic Short Convolutions Improve Transformers", technical
summary page, section Metodologia, Mecanismo, applied per sequence), for every
output: y, dx, dw (head-wise), dz and dU (low-rank; dU is the sum over the
sequences). Integer-valued inputs make every comparison exact.
"""
import subprocess

import numpy as np
import pytest

from dynamic_short_convolutions_amd.synthetic import f32_to_bf16_bits, to_float


def store(a, dt):
    a = np.asarray(a, dtype=np.float32)
    return f32_to_bf16_bits(a) if dt == "bf16" else np.ascontiguousarray(a)


def ints(rng, shape, lo=-3, hi=3):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def packing(rng, B, T, W):
    """Per row: sequence lengths (some shorter than W, some of length 1) filling T."""
    segs, pos = [], np.zeros((B, T), np.int32)
    for b in range(B):
        lens, left = [], T
        while left > 0:
            n = int(min(left, rng.choice([1, 2, W - 1 if W > 1 else 1, W, W + 1, 5, 9, 13])))
            lens.append(n)
            left -= n
        a = 0
        for n in lens:
            pos[b, a:a + n] = np.arange(n)
            segs.append((b, a, n))
            a += n
    return segs, pos


def cut(a, b, s, n):
    return np.ascontiguousarray(a[b:b + 1, s:s + n])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("W,Hc,res", [(1, 2, 1), (2, 1, 0), (3, 4, 1), (4, 8, 1), (6, 2, 0), (8, 4, 1)])
def test_headwise_packed_equals_each_sequence(oracle_mod, dt, W, Hc, res):
    rng = np.random.default_rng(11 * W + Hc)
    B, T, D = 2, 40, 16
    G = D // Hc
    x = store(ints(rng, (B, T, D)), dt)
    w = store(ints(rng, (B, T, G, W)), dt)
    dy = store(ints(rng, (B, T, D)), dt)
    segs, pos = packing(rng, B, T, W)
    y = oracle_mod.fwd(x, w, res, pos=pos)
    dx, dw = oracle_mod.bwd(x, w, dy, res, pos=pos)
    for b, s, n in segs:
        xs, ws, dys = cut(x, b, s, n), cut(w, b, s, n), cut(dy, b, s, n)
        np.testing.assert_array_equal(y[b, s:s + n], oracle_mod.fwd(xs, ws, res)[0])
        dxs, dws = oracle_mod.bwd(xs, ws, dys, res)
        np.testing.assert_array_equal(dx[b, s:s + n], dxs[0])
        np.testing.assert_array_equal(dw[b, s:s + n], dws[0])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("W,R,res", [(1, 2, 0), (3, 1, 1), (4, 3, 0), (7, 2, 1)])
def test_lowrank_packed_equals_each_sequence(oracle_mod, dt, W, R, res):
    rng = np.random.default_rng(5 * W + R)
    B, T, D = 2, 30, 8
    x = store(ints(rng, (B, T, D)), dt)
    z = store(ints(rng, (B, T, R), -2, 2), dt)
    U = store(ints(rng, (R, D * W), -2, 2), dt)
    dy = store(ints(rng, (B, T, D)), dt)
    segs, pos = packing(rng, B, T, W)
    y = oracle_mod.lowrank_fwd(x, z, U, W, res, pos=pos)
    dx, dz, dU = oracle_mod.lowrank_bwd(x, z, U, dy, W, res, pos=pos)
    dU_sum = np.zeros_like(dU)
    for b, s, n in segs:
        xs, zs, dys = cut(x, b, s, n), cut(z, b, s, n), cut(dy, b, s, n)
        np.testing.assert_array_equal(y[b, s:s + n], oracle_mod.lowrank_fwd(xs, zs, U, W, res)[0])
        dxs, dzs, dUs = oracle_mod.lowrank_bwd(xs, zs, U, dys, W, res)
        np.testing.assert_array_equal(dx[b, s:s + n], dxs[0])
        np.testing.assert_array_equal(dz[b, s:s + n], dzs[0])
        dU_sum += dUs
    np.testing.assert_array_equal(dU, dU_sum)


def test_one_sequence_per_row_equals_dense(oracle_mod):
    """pos[t] = t (and any pos[t] >= W-1 once t >= W-1) is the dense operation."""
    rng = np.random.default_rng(3)
    B, T, D, W, R = 2, 17, 8, 4, 3
    x, dy = ints(rng, (B, T, D)), ints(rng, (B, T, D))
    w = ints(rng, (B, T, 4, W))
    z, U = ints(rng, (B, T, R)), ints(rng, (R, D * W))
    pos = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    big = pos + 1000
    for p in (pos, big):
        np.testing.assert_array_equal(oracle_mod.fwd(x, w, 1, pos=p), oracle_mod.fwd(x, w, 1))
        for a, b in zip(oracle_mod.bwd(x, w, dy, 1, pos=p), oracle_mod.bwd(x, w, dy, 1)):
            np.testing.assert_array_equal(a, b)
        for a, b in zip(oracle_mod.lowrank_bwd(x, z, U, dy, W, 0, pos=p), oracle_mod.lowrank_bwd(x, z, U, dy, W, 0)):
            np.testing.assert_array_equal(a, b)


def test_every_token_its_own_sequence(oracle_mod):
    """pos = 0 everywhere keeps tap 0 only: y = (w_0 + residual) x, dx likewise, dw_k = 0 for k > 0."""
    rng = np.random.default_rng(4)
    B, T, D, G, W = 2, 9, 8, 2, 3
    x, dy = ints(rng, (B, T, D)), ints(rng, (B, T, D))
    w = ints(rng, (B, T, G, W))
    pos = np.zeros((B, T), np.int32)
    w0 = np.repeat(w[..., 0], D // G, axis=2).astype(np.float64)
    np.testing.assert_array_equal(oracle_mod.fwd(x, w, 1, pos=pos), (w0 + 1) * x)
    dx, dw = oracle_mod.bwd(x, w, dy, 1, pos=pos)
    np.testing.assert_array_equal(dx, (w0 + 1) * dy)
    assert not dw[..., 1:].any()
    np.testing.assert_array_equal(dw[..., 0], (dy * x).reshape(B, T, G, D // G).sum(-1))


# ------------------------------------------------------------------ planted mistakes are caught

MUTATIONS = [
    ("a tap exists only below the position", "k <= pos[n]", "k < pos[n]"),
    ("head-wise dx ignores positions",
     "if (!tap_on(pos, b * T + s + k, s + k, k)) continue;\n          acc += ld(w,",
     "acc += ld(w,"),
    ("head-wise dx asks step s instead of s+k",
     "if (!tap_on(pos, b * T + s + k, s + k, k)) continue;\n          acc += ld(w,",
     "if (!tap_on(pos, b * T + s, s + k, k)) continue;\n          acc += ld(w,"),
    ("low-rank dx ignores positions",
     "if (!tap_on(pos, b * T + s + k, s + k, k)) continue;\n            acc += omega",
     "acc += omega"),
    ("dU ignores positions", "if (!tap_on(pos, b * T + t, t, k)) continue;\n", ""),
    ("dw ignores positions", "if (tap_on(pos, b * T + t, t, k)) {", "if (t - k >= 0) {"),
]


def _checks(o):
    return [
        lambda: test_headwise_packed_equals_each_sequence(o, "f32", 4, 8, 1),
        lambda: test_lowrank_packed_equals_each_sequence(o, "f32", 4, 3, 0),
        lambda: test_every_token_its_own_sequence(o),
    ]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_varlen_pins_catch_planted_mistake(oracle_mod, tmp_path, name, old, new):
    src = open(oracle_mod.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(lib),
                    str(mutated)], check=True)
    caught = 0
    with oracle_mod.use_library(str(lib)):
        for check in _checks(oracle_mod):
            try:
                check()
            except AssertionError:
                caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"
    for check in _checks(oracle_mod):
        check()
