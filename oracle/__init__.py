"""CPU oracle for the causal dynamic short convolution (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never imports, links or calls it.

``build()`` compiles ``dsc_oracle.c`` (plain C, double accumulation, OpenMP
over output rows) with gcc into ``liboracle.so`` next to it. The functions
below marshal numpy arrays into it; each returns float64 arrays. Inputs are
float32 arrays or bfloat16 bit patterns (uint16 arrays).

``npref`` holds a second, independent NumPy formulation of the same
definitions for tiny shapes, used only to cross-check the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "dsc_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
_lib = None


def build(force: bool = True, out: str | None = None, extra_flags=()) -> str:
    """Compile the oracle library with gcc (no GPU code involved). ``out`` and
    ``extra_flags`` build another copy (e.g. instrumented by the sanitizer tests)."""
    lib = out or LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(SRC):
        tmp = lib + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", *extra_flags, "-o", tmp, SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


def _bind(path: str):
    lib = ctypes.CDLL(path)
    vp, i64, i32, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp, i64, dp]
    lib.oracle_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp, i64, dp, dp]
    lib.oracle_lowrank_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, vp, i64, dp]
    lib.oracle_lowrank_bwd_rows.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32,
                                            vp, i64, dp, dp]
    lib.oracle_lowrank_dU.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp, i64, dp]
    lib.oracle_fwd_w64.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp, i64, dp]
    lib.oracle_bwd_dy64.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp, i64, dp, dp]
    lib.oracle_bwd_w64.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp, i64, dp, dp]
    lib.oracle_decode_step.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, dp, vp]
    lib.oracle_lowrank_decode_step.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, dp, vp]
    lib.oracle_decode_state_from_prefill.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp]
    for f in ("oracle_fwd", "oracle_bwd", "oracle_lowrank_fwd", "oracle_lowrank_bwd_rows",
              "oracle_lowrank_dU", "oracle_bwd_dy64", "oracle_bwd_w64", "oracle_fwd_w64", "oracle_decode_step", "oracle_lowrank_decode_step",
              "oracle_decode_state_from_prefill", "oracle_abi_version", "oracle_get_threads"):
        getattr(lib, f).restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        alt = os.environ.get("DSC_ORACLE_LIB")  # another build of dsc_oracle.c (sanitizer runs)
        if alt:
            _lib = _bind(alt)
        else:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build(force=False)
            _lib = _bind(LIB)
    return _lib


class use_library:
    """Context manager: route every oracle call to another build of dsc_oracle.c
    (the mutation tests use it to check that the pins catch planted mistakes)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _load()
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def _dt(*arrays) -> int:
    kinds = {a.dtype for a in arrays if a is not None}
    if kinds == {np.dtype(np.float32)}:
        return F32
    if kinds == {np.dtype(np.uint16)}:
        return BF16
    raise TypeError(f"oracle inputs must all be float32 or all bf16 bits (uint16); got {kinds}")


def _p(a):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle inputs must be C-contiguous")
    return a.ctypes.data


def _rows(rows, B, T):
    if rows is None:
        return None, B * T
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= B * T):
        raise ValueError("row index out of range")
    return r, r.size


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments")


def _positions(pos, B, T):
    """Token positions within their sequences, [B,T] int32, or None (each row one sequence)."""
    if pos is None:
        return None
    p = np.ascontiguousarray(pos, dtype=np.int32)
    if p.shape != (B, T):
        raise ValueError("pos must be [B, T]")
    return p


def fwd(x, w, residual, rows=None, pos=None):
    """Head-wise forward. x [B,T,D], w [B,T,G,W] -> y [nrows, D] (all tokens: [B,T,D]).
    pos [B,T]: index of each token within its packed sequence (None: one sequence per row)."""
    B, T, D = x.shape
    G, W = w.shape[2], w.shape[3]
    r, n = _rows(rows, B, T)
    q = _positions(pos, B, T)
    y = np.empty((n, D), np.float64)
    _check(_load().oracle_fwd(_p(x), _p(w), _p(q), B, T, D, G, W, int(residual), _dt(x, w), _p(r), n, _p(y)))
    return y.reshape(B, T, D) if rows is None else y


def bwd(x, w, dy, residual, rows=None, want_dx=True, want_dw=True, pos=None):
    """Head-wise backward -> (dx [.., D], dw [.., G, W])."""
    B, T, D = x.shape
    G, W = w.shape[2], w.shape[3]
    r, n = _rows(rows, B, T)
    q = _positions(pos, B, T)
    dx = np.empty((n, D), np.float64) if want_dx else None
    dw = np.empty((n, G, W), np.float64) if want_dw else None
    _check(_load().oracle_bwd(_p(x), _p(w), _p(dy), _p(q), B, T, D, G, W, int(residual), _dt(x, w, dy),
                              _p(r), n, _p(dx), _p(dw)))
    if rows is None:
        dx = dx.reshape(B, T, D) if dx is not None else None
        dw = dw.reshape(B, T, G, W) if dw is not None else None
    return dx, dw


def lowrank_fwd(x, z, U, W, residual, rows=None, pos=None):
    """Low-rank forward. x [B,T,D], z [B,T,R], U [R, D*W] -> y."""
    B, T, D = x.shape
    R = z.shape[2]
    if U.shape != (R, D * W):
        raise ValueError("U must be [R, D*W]")
    r, n = _rows(rows, B, T)
    q = _positions(pos, B, T)
    y = np.empty((n, D), np.float64)
    _check(_load().oracle_lowrank_fwd(_p(x), _p(z), _p(U), _p(q), B, T, D, R, W, int(residual),
                                      _dt(x, z, U), _p(r), n, _p(y)))
    return y.reshape(B, T, D) if rows is None else y


def lowrank_bwd_rows(x, z, U, dy, W, residual, rows=None, want_dx=True, want_dz=True, pos=None):
    """Low-rank per-token gradients -> (dx [.., D], dz [.., R])."""
    B, T, D = x.shape
    R = z.shape[2]
    r, n = _rows(rows, B, T)
    q = _positions(pos, B, T)
    dx = np.empty((n, D), np.float64) if want_dx else None
    dz = np.empty((n, R), np.float64) if want_dz else None
    _check(_load().oracle_lowrank_bwd_rows(_p(x), _p(z), _p(U), _p(dy), _p(q), B, T, D, R, W, int(residual),
                                           _dt(x, z, U, dy), _p(r), n, _p(dx), _p(dz)))
    if rows is None:
        dx = dx.reshape(B, T, D) if dx is not None else None
        dz = dz.reshape(B, T, R) if dz is not None else None
    return dx, dz


def lowrank_dU(x, z, dy, W, cols=None, pos=None):
    """Gradient of U over all tokens -> dU [R, ncols] (all columns: [R, D*W])."""
    B, T, D = x.shape
    R = z.shape[2]
    q = _positions(pos, B, T)
    if cols is None:
        c, n = None, D * W
    else:
        c = np.ascontiguousarray(cols, dtype=np.int64)
        n = c.size
        if n and (c.min() < 0 or c.max() >= D * W):
            raise ValueError("column index out of range")
    dU = np.empty((R, n), np.float64)
    _check(_load().oracle_lowrank_dU(_p(x), _p(z), _p(dy), _p(q), B, T, D, R, W, _dt(x, z, dy), _p(c), n,
                                     _p(dU)))
    return dU


def lowrank_bwd(x, z, U, dy, W, residual, pos=None):
    """All low-rank gradients on every token (small shapes) -> (dx, dz, dU)."""
    dx, dz = lowrank_bwd_rows(x, z, U, dy, W, residual, pos=pos)
    return dx, dz, lowrank_dU(x, z, dy, W, pos=pos)


# ------------------------------------------------------------------ decode step

def _pos(pos, B):
    p = np.ascontiguousarray(pos, dtype=np.int32)
    if p.shape != (B,):
        raise ValueError("pos must be [B] int32")
    return p


def _ring(state, B, W, D, dtype):
    if state.shape != (B, W - 1, D) or state.dtype != dtype:
        raise ValueError("state must be [B, W-1, D] in the inputs' storage type")
    return np.array(state, copy=True, order="C")


def decode_step(x, w, pos, state, residual):
    """Head-wise decode step. x [B,D], w [B,G,W], pos [B] int32, state [B,W-1,D]
    -> (y [B,D] float64, NaN on rows with pos < 0; the updated ring, a new array)."""
    B, D = x.shape
    G, W = w.shape[1], w.shape[2]
    p = _pos(pos, B)
    out = _ring(state, B, W, D, x.dtype)
    y = np.empty((B, D), np.float64)
    _check(_load().oracle_decode_step(_p(x), _p(w), _p(p), _p(state), B, D, G, W, int(residual),
                                      _dt(x, w, state), _p(y), _p(out)))
    return y, out


def lowrank_decode_step(x, z, U, pos, state, W, residual):
    """Low-rank decode step. x [B,D], z [B,R], U [R,D*W] -> (y [B,D], updated ring)."""
    B, D = x.shape
    R = z.shape[1]
    if U.shape != (R, D * W):
        raise ValueError("U must be [R, D*W]")
    p = _pos(pos, B)
    out = _ring(state, B, W, D, x.dtype)
    y = np.empty((B, D), np.float64)
    _check(_load().oracle_lowrank_decode_step(_p(x), _p(z), _p(U), _p(p), _p(state), B, D, R, W,
                                              int(residual), _dt(x, z, U, state), _p(y), _p(out)))
    return y, out


def decode_state_from_prefill(x, lengths, state):
    """Ring after prompts: x [B,T,D], lengths [B] -> the updated ring (a new array)."""
    B, T, D = x.shape
    W = state.shape[1] + 1
    p = _pos(lengths, B)
    out = _ring(state, B, W, D, x.dtype)
    _check(_load().oracle_decode_state_from_prefill(_p(x), _p(p), B, T, D, W, _dt(x, state), _p(out)))
    return out


# ------------------------------------------------------------------ rotary embedding after the convolution

def _as_f64(a):
    """Storage array (float32, bf16 bits as uint16, or float64) -> float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def rope_apply(y, cos, sin, d_rot, head_dim, interleaved, pos=None, inverse=False):
    """Rotary position embedding (RoFormer) on channels [0, d_rot) of y [B,T,D] (float64).

    Those channels form heads of head_dim channels; in each head, pair i (i < head_dim/2)
    is the channels (i, i + head_dim/2) (interleaved=False) or (2i, 2i+1) (interleaved=True),
    and (a, b) becomes (a cos - b sin, a sin + b cos) with cos = cos[p, i], sin = sin[p, i]
    for the token's position p (pos[b,t], or t when pos is None), clamped to the table's
    rows. inverse=True rotates by the opposite angle (the transpose). Other channels pass.
    """
    B, T, D = np.shape(y)
    p = np.tile(np.arange(T, dtype=np.int64), (B, 1)) if pos is None else np.asarray(pos, dtype=np.int64)
    flat = rope_apply_rows(np.reshape(y, (B * T, D)), p.reshape(-1), cos, sin, d_rot, head_dim, interleaved,
                           inverse)
    return flat.reshape(B, T, D)


def rope_apply_rows(y, p, cos, sin, d_rot, head_dim, interleaved, inverse=False):
    """rope_apply on token rows y [n, D] at positions p [n] (the same rotation, row by row)."""
    y = np.array(y, dtype=np.float64, copy=True)
    n, D = y.shape
    n_pos, half = cos.shape
    if 2 * half != head_dim or d_rot % head_dim or d_rot > D or sin.shape != cos.shape:
        raise ValueError("rotary table, head size and rotated channels do not fit")
    p = np.clip(np.asarray(p, dtype=np.int64), 0, n_pos - 1)
    C = np.asarray(cos, dtype=np.float64)[p]
    S = np.asarray(sin, dtype=np.float64)[p]
    if inverse:
        S = -S
    i = np.arange(half)
    for h in range(d_rot // head_dim):
        ia = h * head_dim + (2 * i if interleaved else i)
        ib = ia + (1 if interleaved else half)
        a, b = y[:, ia].copy(), y[:, ib].copy()
        y[:, ia] = a * C - b * S
        y[:, ib] = a * S + b * C
    return y


def fwd_rope(x, w, residual, cos, sin, d_rot, head_dim, interleaved, pos=None, rows=None):
    """Head-wise forward followed by the rotary embedding of its Q and K channels.
    rows: optional flat token indices b*T+t (output [n, D] then)."""
    B, T, D = x.shape
    if rows is None:
        return rope_apply(fwd(x, w, residual, pos=pos), cos, sin, d_rot, head_dim, interleaved, pos=pos)
    r = np.asarray(rows, dtype=np.int64)
    p = (r % T) if pos is None else np.asarray(pos).reshape(-1)[r]
    return rope_apply_rows(fwd(x, w, residual, rows=r, pos=pos), p, cos, sin, d_rot, head_dim, interleaved)


def bwd_rope(x, w, dy, residual, cos, sin, d_rot, head_dim, interleaved, pos=None, rows=None):
    """Gradients (dx, dw) of fwd_rope: the transposed rotation takes dy back to the
    convolution's output, then its backward (dy carried in double). rows as in fwd_rope."""
    B, T, D = x.shape
    G, W = w.shape[2], w.shape[3]
    dyc = np.ascontiguousarray(rope_apply(_as_f64(dy), cos, sin, d_rot, head_dim, interleaved, pos=pos,
                                          inverse=True))
    q = _positions(pos, B, T)
    r, n = _rows(rows, B, T)
    dx = np.empty((n, D), np.float64)
    dw = np.empty((n, G, W), np.float64)
    _check(_load().oracle_bwd_dy64(_p(x), _p(w), _p(dyc), _p(q), B, T, D, G, W, int(residual), _dt(x, w),
                                   _p(r), n, _p(dx), _p(dw)))
    if rows is None:
        return dx.reshape(B, T, D), dw.reshape(B, T, G, W)
    return dx, dw


# ------------------------------------------------------------------ filter generator

def generate_filters(h, Wg, G, W):
    """Head-wise filters from the hidden state (Parametrizacao: a learned linear map of
    the current hidden state): w[b,t,g,k] = sum_j h[b,t,j] * Wg[g*W+k, j], in float64.
    h [B,T,K] and Wg [G*W, K] in a storage type; returns w [B,T,G,W] float64."""
    B, T, K = h.shape
    if Wg.shape != (G * W, K):
        raise ValueError("Wg must be [G*W, K]")
    return np.matmul(_as_f64(h), _as_f64(Wg).T).reshape(B, T, G, W)


def fwd_gen(x, h, Wg, G, W, residual, rows=None, pos=None):
    """Head-wise forward with the filters generated from h: fwd(x, generate_filters(h, Wg))."""
    B, T, D = x.shape
    r, n = _rows(rows, B, T)
    if rows is None:
        w = np.ascontiguousarray(generate_filters(h, Wg, G, W))
    else:  # the filters of the selected steps only (each output reads its own step's filter)
        w = np.zeros((B * T, G, W), np.float64)
        w[r] = generate_filters(np.ascontiguousarray(h.reshape(B * T, -1)[r])[None], Wg, G, W)[0]
    q = _positions(pos, B, T)
    y = np.empty((n, D), np.float64)
    _check(_load().oracle_fwd_w64(_p(x), _p(w), _p(q), B, T, D, G, W, int(residual), _dt(x), _p(r), n, _p(y)))
    return y.reshape(B, T, D) if rows is None else y


def bwd_gen(x, h, Wg, dy, G, W, residual, rows=None, pos=None):
    """Backward of fwd_gen with respect to x and to the generated filters:
    bwd(x, generate_filters(h, Wg), dy) with the filters in float64 -> (dx, dw).
    dx at step s uses the filters of steps s .. s+W-1; dw does not use the filters
    (the gradients of h and Wg are then dw's products with Wg and h)."""
    B, T, D = x.shape
    r, n = _rows(rows, B, T)
    if rows is None:
        w = np.ascontiguousarray(generate_filters(h, Wg, G, W))
    else:  # the filters of the steps the selected outputs read: s .. s+W-1 of the same sequence
        sel = np.array(sorted({rr + k for rr in r.tolist() for k in range(W) if rr % T + k < T}), dtype=np.int64)
        w = np.zeros((B * T, G, W), np.float64)
        if sel.size:
            w[sel] = generate_filters(np.ascontiguousarray(h.reshape(B * T, -1)[sel])[None], Wg, G, W)[0]
    q = _positions(pos, B, T)
    dx = np.empty((n, D), np.float64)
    dw = np.empty((n, G, W), np.float64)
    _check(_load().oracle_bwd_w64(_p(x), _p(w), _p(dy), _p(q), B, T, D, G, W, int(residual), _dt(x, dy), _p(r), n,
                                  _p(dx), _p(dw)))
    if rows is None:
        return dx.reshape(B, T, D), dw.reshape(B, T, G, W)
    return dx, dw
