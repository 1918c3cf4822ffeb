"""Pins of the oracle's decode step (one new token per sequence, inputs of the
previous W-1 steps kept in a ring per sequence) against facts that fix it.

The decode step is the forward definition ("Dynamic Short Convolutions Improve
Transformers", technical summary page, section Metodologia, Mecanismo, with
the two parametrisations and the residual of Posicionamento) evaluated at one
step. So a decode run over a whole sequence must reproduce the forward oracle
(itself pinned by the other pin file) exactly, a constant filter must give
numpy.convolve, and the ring must hold, bit for bit, the last W-1 inputs at
slot s mod (W-1). Slots that belong to steps before 0 are filled with NaN:
the step must never read them. Integer-valued inputs keep every sum exact.
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


def nan_ring(B, W, D, dt):
    return store(np.full((B, W - 1, D), np.nan, np.float32), dt)


def bits_equal(a, b):
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


# ------------------------------------------------------------------ replay of a whole sequence

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("W,Hc,res", [(1, 4, 1), (2, 1, 0), (3, 2, 1), (4, 8, 1), (8, 4, 0)])
def test_headwise_decode_replays_forward(oracle_mod, dt, W, Hc, res):
    rng = np.random.default_rng(100 * W + Hc)
    B, T, D = 3, 12, 16
    G = D // Hc
    x = store(ints(rng, (B, T, D)), dt)
    w = store(ints(rng, (B, T, G, W)), dt)
    y_full = oracle_mod.fwd(x, w, res)
    ring = nan_ring(B, W, D, dt)
    for t in range(T):
        pos = np.full(B, t, np.int32)
        y, ring = oracle_mod.decode_step(np.ascontiguousarray(x[:, t]), np.ascontiguousarray(w[:, t]), pos,
                                         ring, res)
        np.testing.assert_array_equal(y, y_full[:, t], err_msg=f"step {t}")
        for s in range(max(0, t - W + 2), t + 1):  # the ring holds x_s at slot s mod (W-1)
            assert bits_equal(ring[:, s % (W - 1)], x[:, s]), f"step {t}: slot of x_{s}"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("W,R,res", [(1, 2, 1), (3, 1, 0), (4, 3, 1), (8, 2, 1)])
def test_lowrank_decode_replays_forward(oracle_mod, dt, W, R, res):
    rng = np.random.default_rng(7 * W + R)
    B, T, D = 2, 11, 8
    x = store(ints(rng, (B, T, D)), dt)
    z = store(ints(rng, (B, T, R), -2, 2), dt)
    U = store(ints(rng, (R, D * W), -2, 2), dt)
    y_full = oracle_mod.lowrank_fwd(x, z, U, W, res)
    ring = nan_ring(B, W, D, dt)
    for t in range(T):
        pos = np.full(B, t, np.int32)
        y, ring = oracle_mod.lowrank_decode_step(np.ascontiguousarray(x[:, t]), np.ascontiguousarray(z[:, t]),
                                                 U, pos, ring, W, res)
        np.testing.assert_array_equal(y, y_full[:, t], err_msg=f"step {t}")
        for s in range(max(0, t - W + 2), t + 1):
            assert bits_equal(ring[:, s % (W - 1)], x[:, s]), f"step {t}: slot of x_{s}"


# ------------------------------------------------------------------ a library routine

@pytest.mark.parametrize("W", [2, 4, 6])
def test_constant_filter_decode_is_numpy_convolve(oracle_mod, W):
    """Filters constant in time: the decoded outputs form numpy.convolve's causal part."""
    rng = np.random.default_rng(W)
    B, T, D, Hc = 2, 15, 8, 2
    G = D // Hc
    x = store(rng.standard_normal((B, T, D)), "f32")
    v = rng.standard_normal((G, W)).astype(np.float32)
    w_step = np.ascontiguousarray(np.broadcast_to(v, (B, G, W)))
    ring = nan_ring(B, W, D, "f32")
    ys = []
    for t in range(T):
        y, ring = oracle_mod.decode_step(np.ascontiguousarray(x[:, t]), w_step, np.full(B, t, np.int32), ring, 0)
        ys.append(y)
    ys = np.stack(ys, axis=1)
    for b in range(B):
        for c in range(D):
            ref = np.convolve(x[b, :, c].astype(np.float64), v[c // Hc].astype(np.float64))[:T]
            np.testing.assert_allclose(ys[b, :, c], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ prompts, mixed positions, idle rows

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("W", [2, 4, 7])
def test_prefill_then_step_at_mixed_positions(oracle_mod, dt, W):
    """Each row at its own position t_b (0, short, long): the ring built from its
    prompt x[b, :t_b] and one step give the forward output at (b, t_b)."""
    rng = np.random.default_rng(31 + W)
    T, D, Hc = 20, 16, 4
    t_b = np.array([0, 1, W - 2, W - 1, W, 13, T - 1], np.int32)
    B = t_b.size
    G = D // Hc
    x = store(ints(rng, (B, T, D)), dt)
    w = store(ints(rng, (B, T, G, W)), dt)
    y_full = oracle_mod.fwd(x, w, 1)
    ring = oracle_mod.decode_state_from_prefill(x, t_b, nan_ring(B, W, D, dt))
    rows = np.arange(B)
    y, ring2 = oracle_mod.decode_step(np.ascontiguousarray(x[rows, t_b]), np.ascontiguousarray(w[rows, t_b]), t_b,
                                      ring, 1)
    np.testing.assert_array_equal(y, y_full[rows, t_b])
    for b in range(B):  # after the step the ring holds x_{t_b - W + 2} .. x_{t_b}
        for s in range(max(0, t_b[b] - W + 2), t_b[b] + 1):
            assert bits_equal(ring2[b, s % (W - 1)], x[b, s])


def test_prefill_lengths_are_clamped(oracle_mod):
    rng = np.random.default_rng(3)
    B, T, D, W = 3, 5, 8, 4
    x = store(ints(rng, (B, T, D)), "f32")
    ring0 = store(ints(rng, (B, W - 1, D), 10, 20), "f32")
    ring = oracle_mod.decode_state_from_prefill(x, np.array([-4, 0, 99], np.int32), ring0)
    assert bits_equal(ring[0], ring0[0]) and bits_equal(ring[1], ring0[1])  # nothing consumed
    for s in range(T - W + 1, T):  # a length past T counts as T
        assert bits_equal(ring[2, s % (W - 1)], x[2, s])


def test_idle_rows_are_left_alone(oracle_mod):
    rng = np.random.default_rng(4)
    B, D, G, W = 4, 8, 2, 3
    x = store(ints(rng, (B, D)), "bf16")
    w = store(ints(rng, (B, G, W)), "bf16")
    ring0 = store(ints(rng, (B, W - 1, D)), "bf16")
    pos = np.array([5, -1, 0, -7], np.int32)
    y, ring = oracle_mod.decode_step(x, w, pos, ring0, 1)
    assert np.isnan(y[[1, 3]]).all() and np.isfinite(y[[0, 2]]).all()
    assert bits_equal(ring[[1, 3]], ring0[[1, 3]])
    # the active rows: the first step of a sequence reads no ring slot
    xf, wf = to_float(x), to_float(w)
    np.testing.assert_array_equal(y[2], (wf[2, np.arange(D) // (D // G), 0] + 1) * xf[2])


def test_width_one_keeps_no_ring(oracle_mod):
    rng = np.random.default_rng(5)
    B, D = 2, 8
    x = store(rng.standard_normal((B, D)), "f32")
    w = store(np.ones((B, 4, 1)), "f32")
    y, ring = oracle_mod.decode_step(x, w, np.array([0, 9], np.int32), np.zeros((B, 0, D), np.float32), 1)
    np.testing.assert_array_equal(y, 2 * x.astype(np.float64))
    assert ring.shape == (B, 0, D)


# ------------------------------------------------------------------ planted mistakes are caught

MUTATIONS = [
    ("decode reads the slot one step late", "(b * S + (t - k) % S)", "(b * S + (t - k + 1) % S)"),
    ("decode stores the new input one slot ahead",
     "(b * S + t % S) * D) * e, (const char*)x + (size_t)(b * D) * e",
     "(b * S + (t + 1) % S) * D) * e, (const char*)x + (size_t)(b * D) * e"),
    ("decode reads slots of steps before 0", "if (t - k < 0) break;\n      const double xv", "const double xv"),
    ("decode drops the residual", "if (residual) acc += ld(x, b * D + c, dt);", ""),
    ("decode maps channel to head by c % G", "ld(w, (b * G + c / Hc) * W + k, dt)", "ld(w, (b * G + c % G) * W + k, dt)"),
    ("low-rank decode uses the first row's z", "lowrank_filter(z, U, b, 0, 1, D, R, W, dt, f);",
     "lowrank_filter(z, U, 0, 0, 1, D, R, W, dt, f);"),
    ("prefill leaves out the last prompt token", "s < n; ++s)", "s < n - 1; ++s)"),
]


def _decode_checks(o):
    return [
        lambda: test_headwise_decode_replays_forward(o, "f32", 4, 8, 1),
        lambda: test_headwise_decode_replays_forward(o, "bf16", 3, 2, 1),
        lambda: test_lowrank_decode_replays_forward(o, "f32", 4, 3, 1),
        lambda: test_constant_filter_decode_is_numpy_convolve(o, 4),
        lambda: test_prefill_then_step_at_mixed_positions(o, "f32", 4),
        lambda: test_prefill_lengths_are_clamped(o),
        lambda: test_idle_rows_are_left_alone(o),
    ]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_decode_pins_catch_planted_mistake(oracle_mod, tmp_path, name, old, new):
    src = open(oracle_mod.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(lib),
                    str(mutated)], check=True)
    caught = 0
    with oracle_mod.use_library(str(lib)):
        for check in _decode_checks(oracle_mod):
            try:
                check()
            except AssertionError:
                caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"
    for check in _decode_checks(oracle_mod):
        check()
