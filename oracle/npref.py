"""Second, independent formulation of the oracle in NumPy (tiny shapes only).

Test infrastructure. Where the C oracle loops over single output elements,
this file works on whole tensors with time shifts: shift(x, k)[b,t] = x[b,t-k]
(zero for t < k). It exists only to cross-check the C code on random tiny
inputs; it is not one of the oracle's pins.

Source: "Dynamic Short Convolutions Improve Transformers" (technical summary
page), section Metodologia (Mecanismo, Parametrizacao 1 and 2, Posicionamento).
"""
from __future__ import annotations

import numpy as np


def shift(a: np.ndarray, k: int) -> np.ndarray:
    """a[b, t-k, ...] along axis 1, zero where t < k."""
    out = np.zeros_like(a)
    if k < a.shape[1]:
        out[:, k:] = a[:, : a.shape[1] - k]
    return out


def unshift(a: np.ndarray, k: int) -> np.ndarray:
    """a[b, t+k, ...] along axis 1, zero where t+k >= T (the adjoint of shift)."""
    out = np.zeros_like(a)
    if k < a.shape[1]:
        out[:, : a.shape[1] - k] = a[:, k:]
    return out


def per_channel(w: np.ndarray, Hc: int) -> np.ndarray:
    """[B,T,G,W] tied filters -> [B,T,D,W] per-channel filters."""
    return np.repeat(w, Hc, axis=2)


def fwd(x, w, residual):
    B, T, D = x.shape
    G, W = w.shape[2:]
    wc = per_channel(w, D // G)
    y = residual * x.copy()
    for k in range(W):
        y += wc[..., k] * shift(x, k)
    return y


def bwd(x, w, dy, residual):
    B, T, D = x.shape
    G, W = w.shape[2:]
    Hc = D // G
    wc = per_channel(w, Hc)
    dx = residual * dy.copy()
    dw = np.zeros((B, T, G, W))
    for k in range(W):
        dx += unshift(wc[..., k] * dy, k)
        dw[..., k] = (dy * shift(x, k)).reshape(B, T, G, Hc).sum(-1)
    return dx, dw


def lowrank_filters(z, U, D, W):
    B, T, R = z.shape
    return (z.reshape(B * T, R) @ U).reshape(B, T, D, W)


def lowrank_fwd(x, z, U, W, residual):
    D = x.shape[2]
    return fwd(x, lowrank_filters(z, U, D, W), residual)


def lowrank_bwd(x, z, U, dy, W, residual):
    B, T, D = x.shape
    R = z.shape[2]
    dx, dwfull = bwd(x, lowrank_filters(z, U, D, W), dy, residual)
    g = dwfull.reshape(B * T, D * W)
    dz = (g @ U.T).reshape(B, T, R)
    dU = z.reshape(B * T, R).T @ g
    return dx, dz, dU
