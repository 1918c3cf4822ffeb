"""Pins of the oracle's rotary embedding after the convolution (the QKV placement:
the convolution runs on Q, K and V before the rotary embedding, "Dynamic Short
Convolutions Improve Transformers", technical summary page, section Metodologia,
Posicionamento).

The rotation itself follows the rotary position embedding of RoFormer (Su et al.):
each pair of a head's channels is rotated by its index's angle at the token's
position. Pins: position 0 is the identity; the closed form on unit vectors
against math.cos/math.sin; each pair's norm is kept and the inverse undoes it;
scores between rotated vectors depend only on the distance of their positions;
the two pairings are one channel permutation apart; the fused backward equals
torch autograd (float64, CPU) of the same forward, and satisfies the adjoint
identity for x and for w; planted mistakes are caught.
"""
import math

import numpy as np
import pytest

from dynamic_short_convolutions_amd.synthetic import rope_table


def ints(rng, shape, lo=-3, hi=3):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


@pytest.mark.parametrize("inter", [False, True])
def test_position_zero_is_identity(oracle_mod, inter):
    cos, sin = rope_table(8, 16)
    y = np.random.default_rng(0).standard_normal((2, 1, 48))
    np.testing.assert_array_equal(oracle_mod.rope_apply(y, cos, sin, 32, 16, inter), y)


@pytest.mark.parametrize("inter", [False, True])
def test_closed_form_on_unit_vectors(oracle_mod, inter):
    """Unit vector on the first channel of pair i, at position p: the pair becomes
    (cos(p*theta_i), sin(p*theta_i)) with theta_i = 10000^(-2i/hd)."""
    hd, p = 8, 5
    cos, sin = rope_table(16, hd)
    for i in range(hd // 2):
        a, b = (2 * i, 2 * i + 1) if inter else (i, i + hd // 2)
        y = np.zeros((1, p + 1, hd))
        y[0, p, a] = 1.0
        r = oracle_mod.rope_apply(y, cos, sin, hd, hd, inter)
        th = p * 10000.0 ** (-2.0 * i / hd)
        assert abs(r[0, p, a] - math.cos(th)) < 1e-7 and abs(r[0, p, b] - math.sin(th)) < 1e-7
        others = np.delete(r[0, p], [a, b])
        assert not others.any()


@pytest.mark.parametrize("inter", [False, True])
def test_norm_kept_and_inverse(oracle_mod, inter):
    rng = np.random.default_rng(1)
    cos, sin = rope_table(64, 32)
    y = rng.standard_normal((2, 40, 96))
    pos = rng.integers(0, 64, size=(2, 40)).astype(np.int32)
    r = oracle_mod.rope_apply(y, cos, sin, 64, 32, inter, pos=pos)
    np.testing.assert_array_equal(r[..., 64:], y[..., 64:])          # channels past d_rot pass
    back = oracle_mod.rope_apply(r, cos, sin, 64, 32, inter, pos=pos, inverse=True)
    np.testing.assert_allclose(back, y, rtol=0, atol=1e-6)
    idx = np.arange(16)
    for h in range(2):
        ia = h * 32 + (2 * idx if inter else idx)
        ib = ia + (1 if inter else 16)
        np.testing.assert_allclose(r[..., ia] ** 2 + r[..., ib] ** 2, y[..., ia] ** 2 + y[..., ib] ** 2,
                                   rtol=1e-6, atol=1e-12)


def test_scores_depend_on_distance_only(oracle_mod):
    """<R_p q, R_s k> = <R_{p+d} q, R_{s+d} k>: the property the embedding exists for."""
    rng = np.random.default_rng(2)
    hd = 64
    cos, sin = rope_table(512, hd)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)

    def rot(v, p):
        y = np.zeros((1, 1, hd))
        y[0, 0] = v
        return oracle_mod.rope_apply(y, cos, sin, hd, hd, False, pos=np.array([[p]], np.int32))[0, 0]

    for p, s_, d in [(10, 3, 100), (200, 250, 37), (0, 7, 300)]:
        assert abs(rot(q, p) @ rot(k, s_) - rot(q, p + d) @ rot(k, s_ + d)) < 1e-4


def test_pairings_are_a_permutation_apart(oracle_mod):
    rng = np.random.default_rng(3)
    hd = 16
    cos, sin = rope_table(32, hd)
    y = rng.standard_normal((2, 20, 2 * hd))
    half = np.arange(hd // 2)
    perm = np.empty(hd, np.int64)                       # interleaved channel -> half-layout channel
    perm[0::2], perm[1::2] = half, half + hd // 2
    full = np.concatenate([perm, hd + perm])
    r_half = oracle_mod.rope_apply(y, cos, sin, 2 * hd, hd, False)
    r_inter = oracle_mod.rope_apply(y[..., full], cos, sin, 2 * hd, hd, True)
    np.testing.assert_array_equal(r_inter, r_half[..., full])


@pytest.mark.parametrize("inter", [False, True])
@pytest.mark.parametrize("packed", [False, True])
def test_fused_backward_matches_torch_autograd(oracle_mod, inter, packed):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    B, T, D, Hc, W, hd, d_rot = 2, 23, 48, 4, 4, 16, 32
    G = D // Hc
    cos, sin = rope_table(32, hd)
    x, w, dy = ints(rng, (B, T, D)), ints(rng, (B, T, G, W)), ints(rng, (B, T, D))
    pos = None
    if packed:
        pos = np.concatenate([np.arange(9), np.arange(14)]).astype(np.int32)[None].repeat(B, 0)
    dx, dw = oracle_mod.bwd_rope(x, w, dy, 1, cos, sin, d_rot, hd, inter, pos=pos)
    y = oracle_mod.fwd_rope(x, w, 1, cos, sin, d_rot, hd, inter, pos=pos)

    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    p = torch.arange(T).repeat(B, 1) if pos is None else torch.tensor(pos, dtype=torch.int64)
    taps = torch.repeat_interleave(wt, Hc, dim=2)                         # [B,T,D,W]
    out = xt.clone()
    for k in range(W):
        xs = torch.nn.functional.pad(xt, (0, 0, k, 0))[:, :T]             # x[t-k]
        on = (p >= k).unsqueeze(-1).to(torch.float64)                    # tap k exists
        out = out + taps[..., k] * xs * on
    C = torch.tensor(cos, dtype=torch.float64)[p]
    S = torch.tensor(sin, dtype=torch.float64)[p]
    i = torch.arange(hd // 2)
    res = out.clone()
    for h in range(d_rot // hd):
        ia = h * hd + (2 * i if inter else i)
        ib = ia + (1 if inter else hd // 2)
        a, b = out[..., ia], out[..., ib]
        res[..., ia] = a * C - b * S
        res[..., ib] = a * S + b * C
    np.testing.assert_allclose(y, res.detach().numpy(), rtol=1e-12, atol=1e-9)
    res.backward(torch.tensor(dy, dtype=torch.float64))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-9)


def test_fused_backward_adjoint_identity(oracle_mod):
    """The forward is linear in x and in w: <dy, f(x + e)> - <dy, f(x)> = <dx, e>, likewise for w."""
    rng = np.random.default_rng(5)
    B, T, D, Hc, W, hd = 1, 30, 32, 8, 3, 16
    cos, sin = rope_table(64, hd)
    x, w, dy = ints(rng, (B, T, D)), ints(rng, (B, T, D // Hc, W)), ints(rng, (B, T, D))
    ex, ew = ints(rng, (B, T, D)), ints(rng, (B, T, D // Hc, W))
    f = lambda xx, ww: oracle_mod.fwd_rope(xx, ww, 0, cos, sin, D, hd, False)
    dx, dw = oracle_mod.bwd_rope(x, w, dy, 0, cos, sin, D, hd, False)
    base = np.sum(dy * f(x, w))
    assert abs(np.sum(dy * f(x + ex, w)) - base - np.sum(dx * ex)) < 1e-6 * (1 + abs(base))
    assert abs(np.sum(dy * f(x, w + ew)) - base - np.sum(dw * ew)) < 1e-6 * (1 + abs(base))


# ------------------------------------------------------------------ planted mistakes are caught

def _mutant(kind):
    """A rope_apply with one plausible mistake planted."""
    def rope_apply(y, cos, sin, d_rot, head_dim, interleaved, pos=None, inverse=False):
        y = np.array(y, dtype=np.float64, copy=True)
        B, T, D = y.shape
        n_pos, half = cos.shape
        p = np.tile(np.arange(T), (B, 1)) if pos is None else np.asarray(pos, dtype=np.int64)
        p = np.clip(p, 0, n_pos - 1)
        if kind == "positions ignored":
            p = np.tile(np.arange(T), (B, 1))
        C, S = cos.astype(np.float64)[p], sin.astype(np.float64)[p]
        if inverse and kind != "backward rotates forward":
            S = -S
        i = np.arange(half)
        for h in range(d_rot // head_dim):
            ia = h * head_dim + (2 * i if interleaved else i)
            ib = ia + (1 if interleaved else half)
            if kind == "wrong partner":
                ib = h * head_dim + ((2 * i + 1) if interleaved else (half + (i + 1) % half))
            a, b = y[:, :, ia].copy(), y[:, :, ib].copy()
            sgn = -1.0 if kind == "sign flip" else 1.0
            y[:, :, ia] = a * C - sgn * b * S
            y[:, :, ib] = sgn * a * S + b * C
        return y
    return rope_apply


@pytest.mark.parametrize("kind", ["sign flip", "wrong partner", "backward rotates forward", "positions ignored"])
def test_rope_pins_catch_planted_mistake(oracle_mod, monkeypatch, kind):
    monkeypatch.setattr(oracle_mod, "rope_apply", _mutant(kind))
    checks = [
        lambda: test_closed_form_on_unit_vectors(oracle_mod, False),
        lambda: test_norm_kept_and_inverse(oracle_mod, False),
        lambda: test_fused_backward_matches_torch_autograd(oracle_mod, False, True),
        lambda: test_fused_backward_adjoint_identity(oracle_mod),
    ]
    caught = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            caught += 1
    assert caught > 0, kind
