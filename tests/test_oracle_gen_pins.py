"""Pins of the oracle's filter generator (head-wise filters produced from the hidden
state by a learned linear map, "Dynamic Short Convolutions Improve Transformers",
technical summary page, section Metodologia, Parametrizacao, with head-wise tying).

fwd_gen composes the generator w = h . Wg^T (Wg in the [G*W, K] layout of a linear
layer's weight) with the head-wise forward. Pins: with integer inputs the generated
filters are exact, so fwd_gen equals the already pinned forward on the
materialised filters; a one-hot generator row copies one hidden channel into one
tap; the output is linear in h; torch's matmul agrees on the generated filters;
planted mistakes are caught.
"""
import numpy as np
import pytest

from dynamic_short_convolutions_amd.synthetic import f32_to_bf16_bits


def store(a, dt):
    a = np.asarray(a, dtype=np.float32)
    return f32_to_bf16_bits(a) if dt == "bf16" else np.ascontiguousarray(a)


def ints(rng, shape, lo=-2, hi=2):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("W,Hc,K", [(1, 8, 16), (3, 2, 32), (4, 8, 64), (8, 16, 32)])
def test_equals_forward_on_materialised_filters(oracle_mod, dt, W, Hc, K):
    rng = np.random.default_rng(W * 100 + K)
    B, T, D = 2, 19, 32
    G = D // Hc
    x, h, Wg = store(ints(rng, (B, T, D)), dt), store(ints(rng, (B, T, K)), dt), store(ints(rng, (G * W, K)), dt)
    w = oracle_mod.generate_filters(h, Wg, G, W)       # small integers: exact, and exact in bf16
    w_store = store(w.astype(np.float32), dt)
    for res in (0, 1):
        np.testing.assert_array_equal(oracle_mod.fwd_gen(x, h, Wg, G, W, res), oracle_mod.fwd(x, w_store, res))
    # packed sequences: the same masks as the forward with positions (pinned per sequence)
    pos = np.zeros((B, T), np.int32)
    for b in range(B):
        starts = [0] + sorted(rng.choice(np.arange(1, T), size=3, replace=False).tolist())
        for i, s0 in enumerate(starts):
            s1 = starts[i + 1] if i + 1 < len(starts) else T
            pos[b, s0:s1] = np.arange(s1 - s0)
    np.testing.assert_array_equal(oracle_mod.fwd_gen(x, h, Wg, G, W, 1, pos=pos), oracle_mod.fwd(x, w_store, 1, pos=pos))


def test_one_hot_generator_row(oracle_mod):
    """Wg[g*W+k] = e_j: tap k of head g is hidden channel j."""
    rng = np.random.default_rng(1)
    B, T, K, G, W = 1, 7, 8, 2, 3
    h = rng.standard_normal((B, T, K)).astype(np.float32)
    Wg = np.zeros((G * W, K), np.float32)
    Wg[1 * W + 2, 5] = 1.0
    w = oracle_mod.generate_filters(h, Wg, G, W)
    assert np.array_equal(w[..., 1, 2], h[..., 5].astype(np.float64))
    w[..., 1, 2] = 0
    assert not w.any()


def test_linear_in_h(oracle_mod):
    rng = np.random.default_rng(2)
    B, T, D, K, G, W = 2, 11, 16, 8, 2, 4
    x, Wg = ints(rng, (B, T, D)), ints(rng, (G * W, K))
    h1, h2 = ints(rng, (B, T, K)), ints(rng, (B, T, K))
    y1 = oracle_mod.fwd_gen(x, h1, Wg, G, W, 0)
    y2 = oracle_mod.fwd_gen(x, h2, Wg, G, W, 0)
    y12 = oracle_mod.fwd_gen(x, (h1 + h2).astype(np.float32), Wg, G, W, 0)
    np.testing.assert_array_equal(y12, y1 + y2)


def test_generator_matches_torch_matmul(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    h = rng.standard_normal((2, 5, 24)).astype(np.float32)
    Wg = rng.standard_normal((12, 24)).astype(np.float32)
    ref = torch.nn.functional.linear(torch.tensor(h, dtype=torch.float64), torch.tensor(Wg, dtype=torch.float64))
    np.testing.assert_allclose(oracle_mod.generate_filters(h, Wg, 3, 4), ref.numpy().reshape(2, 5, 3, 4),
                               rtol=1e-13, atol=1e-13)


def test_generator_pins_catch_planted_mistakes(oracle_mod, monkeypatch):
    """A generator that swaps the roles of head and tap, or that drops the last hidden
    channel, fails the pins that tie it to torch and to a one-hot row."""
    real = oracle_mod.generate_filters

    def swapped(h, Wg, G, W):
        return np.ascontiguousarray(real(h, Wg, G, W).reshape(h.shape[0], h.shape[1], W, G).transpose(0, 1, 3, 2))

    def short(h, Wg, G, W):
        h2 = np.array(h, copy=True)
        h2[..., -1] = 0
        return real(h2, Wg, G, W)

    for mutant in (swapped, short):
        monkeypatch.setattr(oracle_mod, "generate_filters", mutant)
        caught = 0
        for check in (test_one_hot_generator_row, test_generator_matches_torch_matmul):
            try:
                check(oracle_mod)
            except AssertionError:
                caught += 1
        assert caught > 0, mutant.__name__
    monkeypatch.setattr(oracle_mod, "generate_filters", real)


def test_c_reads_double_filters(oracle_mod, tmp_path):
    """The C forward must read the generated filters as double: reading them as the
    inputs' storage type (a planted mistake) breaks the materialised-filter pin."""
    import subprocess

    src = open(oracle_mod.SRC).read()
    old = "return fwd_impl(x, w, pos, B, T, D, G, W, residual, dt, ORACLE_F64, rows, nrows, y);"
    assert src.count(old) == 1
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, "return fwd_impl(x, w, pos, B, T, D, G, W, residual, dt, dt, rows, nrows, y);"))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(lib), str(mutated)],
                   check=True)
    with oracle_mod.use_library(str(lib)):
        with pytest.raises(AssertionError):
            test_equals_forward_on_materialised_filters(oracle_mod, "f32", 4, 8, 64)


# ---------------------------------------------------------------- backward with generated filters
# bwd_gen is the chain rule through the forward with generated filters, with respect
# to x and to the filters: dx reads the generated filters of steps s .. s+W-1 (in
# double), dw is dy * x summed over each head and does not involve the generator.

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("W,Hc,K", [(1, 8, 16), (3, 2, 32), (4, 8, 64), (8, 16, 32)])
def test_bwd_equals_backward_on_materialised_filters(oracle_mod, dt, W, Hc, K):
    rng = np.random.default_rng(W * 200 + K)
    B, T, D = 2, 19, 32
    G = D // Hc
    x, dy = store(ints(rng, (B, T, D)), dt), store(ints(rng, (B, T, D)), dt)
    h, Wg = store(ints(rng, (B, T, K)), dt), store(ints(rng, (G * W, K)), dt)
    w_store = store(oracle_mod.generate_filters(h, Wg, G, W).astype(np.float32), dt)  # exact
    for res in (0, 1):
        dx, dw = oracle_mod.bwd_gen(x, h, Wg, dy, G, W, res)
        dx_ref, dw_ref = oracle_mod.bwd(x, w_store, dy, res)
        np.testing.assert_array_equal(dx, dx_ref)
        np.testing.assert_array_equal(dw, dw_ref)
    # selected rows equal the full computation; packed sequences use the forward's masks
    rows = np.array([0, 1, T - 1, T, 2 * T - 2, 2 * T - 1])
    dxr, dwr = oracle_mod.bwd_gen(x, h, Wg, dy, G, W, 1, rows=rows)
    np.testing.assert_array_equal(dxr, dx.reshape(B * T, D)[rows])
    np.testing.assert_array_equal(dwr, dw.reshape(B * T, G, W)[rows])
    pos = np.zeros((B, T), np.int32)
    for b in range(B):
        for s0, s1 in ((0, 5), (5, 6), (6, T)):
            pos[b, s0:s1] = np.arange(s1 - s0)
    dxp, dwp = oracle_mod.bwd_gen(x, h, Wg, dy, G, W, 1, pos=pos)
    dxp_ref, dwp_ref = oracle_mod.bwd(x, w_store, dy, 1, pos=pos)
    np.testing.assert_array_equal(dxp, dxp_ref)
    np.testing.assert_array_equal(dwp, dwp_ref)


def test_bwd_dw_does_not_involve_the_generator(oracle_mod):
    rng = np.random.default_rng(5)
    B, T, D, K, G, W = 2, 13, 16, 8, 2, 4
    x, dy = ints(rng, (B, T, D)), ints(rng, (B, T, D))
    _, dw1 = oracle_mod.bwd_gen(x, ints(rng, (B, T, K)), ints(rng, (G * W, K)), dy, G, W, 1)
    _, dw2 = oracle_mod.bwd_gen(x, ints(rng, (B, T, K)), ints(rng, (G * W, K)), dy, G, W, 0)
    np.testing.assert_array_equal(dw1, dw2)


def test_bwd_adjoint_of_forward(oracle_mod):
    """y = fwd_gen(x) is linear in x (residual 0): <dy, fwd_gen(v)> = <dx, v> for any v,
    which ties dx to the pinned forward with the same generated filters."""
    rng = np.random.default_rng(6)
    B, T, D, K, G, W = 2, 17, 24, 16, 3, 4
    h = rng.standard_normal((B, T, K)).astype(np.float32)
    Wg = rng.standard_normal((G * W, K)).astype(np.float32)
    dy = rng.standard_normal((B, T, D)).astype(np.float32)
    v = rng.standard_normal((B, T, D)).astype(np.float32)
    dx, _ = oracle_mod.bwd_gen(v, h, Wg, dy, G, W, 0)
    lhs = float(np.sum(dy.astype(np.float64) * oracle_mod.fwd_gen(v, h, Wg, G, W, 0)))
    rhs = float(np.sum(dx * v.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))


def test_bwd_matches_autograd(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    B, T, D, K, G, W = 2, 10, 16, 8, 4, 3
    Hc = D // G
    x = rng.standard_normal((B, T, D)).astype(np.float32)
    h = rng.standard_normal((B, T, K)).astype(np.float32)
    Wg = rng.standard_normal((G * W, K)).astype(np.float32)
    dy = rng.standard_normal((B, T, D)).astype(np.float32)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.nn.functional.linear(torch.tensor(h, dtype=torch.float64),
                                    torch.tensor(Wg, dtype=torch.float64)).reshape(B, T, G, W)
    wt = wt.detach().requires_grad_(True)
    y = xt.clone()  # residual 1
    for k in range(W):
        shifted = torch.nn.functional.pad(xt, (0, 0, k, 0))[:, :T]  # x[t-k], zero before t = 0
        y = y + wt[..., k].repeat_interleave(Hc, dim=2) * shifted
    y.backward(torch.tensor(dy, dtype=torch.float64))
    dx, dw = oracle_mod.bwd_gen(x, h, Wg, dy, G, W, 1)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_c_backward_reads_double_filters(oracle_mod, tmp_path):
    """Planted mistakes in the C backward with double filters: reading them as the
    inputs' storage type, or taking the filter of step s for every tap (instead of
    s+k), each break a pin above."""
    import subprocess

    src = open(oracle_mod.SRC).read()
    good = "return bwd_impl(x, w, dy, pos, B, T, D, G, W, residual, dt, ORACLE_F64, dt, rows, nrows, dx, dw);"
    tap = "acc += ld(w, ((b * T + s + k) * G + h) * W + k, w_dt) * ld(dy, (b * T + s + k) * D + c, dy_dt);"
    assert src.count(good) == 1 and src.count(tap) == 1
    mutants = [src.replace(good, good.replace("ORACLE_F64, dt, rows", "dt, dt, rows")),
               src.replace(tap, tap.replace("((b * T + s + k) * G + h) * W + k", "((b * T + s) * G + h) * W + k"))]
    for i, text in enumerate(mutants):
        mutated = tmp_path / f"mutant{i}.c"
        mutated.write_text(text)
        lib = tmp_path / f"libmutant{i}.so"
        subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(lib), str(mutated)],
                       check=True)
        with oracle_mod.use_library(str(lib)):
            caught = 0
            for check in (lambda: test_bwd_equals_backward_on_materialised_filters(oracle_mod, "f32", 4, 8, 64),
                          lambda: test_bwd_adjoint_of_forward(oracle_mod)):
                try:
                    check()
                except AssertionError:
                    caught += 1
            assert caught > 0, f"mutant {i} not caught"
