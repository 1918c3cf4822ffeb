"""Seeded synthetic workloads for the causal dynamic short convolution.

This module only describes shapes and draws random numbers. It holds none of
the operation's arithmetic, so both sides of every parity check (the GPU
library and the CPU oracle) can take their inputs from it.

Every tensor is drawn i.i.d. Gaussian from numpy's PCG64 generator seeded
with ``seed``, in a fixed order (x, then w or z then U, then dy), as float32,
then stored either as float32 or as bfloat16 bit patterns (uint16, rounded to
nearest-even). The workloads stand in for the language-model pretraining
activations that the method's page trains on (Nemotron-CC), which are not
available here.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("f32", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One problem instance of the operation, described by its sizes only."""

    name: str
    kind: str            # "headwise" (tied filters, w given) or "lowrank" (w = z.U)
    B: int
    T: int
    D: int
    W: int
    residual: int
    dtype: str           # "f32" or "bf16": the storage type of every tensor
    Hc: int = 0          # channels per head (headwise)
    R: int = 0           # rank (lowrank)
    x_std: float = 1.0
    w_std: float = 0.5   # headwise filters
    z_std: float = 1.0   # lowrank
    U_std: float = 0.0   # lowrank; set per workload
    dy_std: float = 1.0
    backward: bool = True
    packed_mean: int = 0  # > 0: each row packs sequences of this mean length (positions pos[B,T])
    rope_head_dim: int = 0    # > 0: rotary embedding of channels [0, rope_d_rot) after the convolution
    rope_d_rot: int = 0
    rope_interleaved: int = 0
    gen_hidden: int = 0       # > 0: filters generated in the kernel from a hidden state of this width

    @property
    def G(self) -> int:
        return self.D // self.Hc if self.kind == "headwise" else self.D

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five problem sizes the library is measured and checked on.
WORKLOADS = {
    # x[1,256,64] fp32, tied filters w[1,256,8,4] (8 channels per filter), residual, forward only.
    "tiny_headwise_f32": Workload("tiny_headwise_f32", "headwise", B=1, T=256, D=64, W=4,
                                  residual=1, dtype="f32", Hc=8, backward=False),
    # Q,K,V projections of a ~2B model concatenated: D = 3*2048, 8 channels per filter.
    "qkv_headwise_bf16": Workload("qkv_headwise_bf16", "headwise", B=8, T=4096, D=3 * 2048, W=4,
                                  residual=1, dtype="bf16", Hc=8),
    # Fused low-rank generator: R=32, W=4 on D=2048, U ~ N(0, 1/(R*W)).
    "lowrank_bf16": Workload("lowrank_bf16", "lowrank", B=8, T=4096, D=2048, W=4, residual=0,
                             dtype="bf16", R=32, U_std=1.0 / math.sqrt(32 * 4)),
    # Convolution after every linear layer, SwiGLU intermediate width: D=8192, 16 channels per filter.
    "alllinear_headwise_bf16": Workload("alllinear_headwise_bf16", "headwise", B=8, T=4096, D=8192,
                                        W=4, residual=1, dtype="bf16", Hc=16),
    # Long sequence, wide kernel: T=65536, W=8, R=64, U ~ N(0, 1/(R*W)).
    "longseq_lowrank_bf16": Workload("longseq_lowrank_bf16", "lowrank", B=1, T=65536, D=4096, W=8,
                                     residual=0, dtype="bf16", R=64, U_std=1.0 / math.sqrt(64 * 8)),
}

# Packed-sequence variants: rows of 4096 tokens filled with documents of mean length
# 800 tokens (a stand-in for packed pretraining documents), positions restart at each
# document start.
WORKLOADS["packed_qkv_headwise_bf16"] = WORKLOADS["qkv_headwise_bf16"].with_(name="packed_qkv_headwise_bf16",
                                                                           packed_mean=800)
WORKLOADS["packed_lowrank_bf16"] = WORKLOADS["lowrank_bf16"].with_(name="packed_lowrank_bf16", packed_mean=800)
# The QKV layer with the rotary embedding fused after the convolution: heads of 128
# channels, Q and K (the first 2 * 2048 channels) rotated, pairs (i, i + 64).
WORKLOADS["rope_qkv_headwise_bf16"] = WORKLOADS["qkv_headwise_bf16"].with_(
    name="rope_qkv_headwise_bf16", rope_head_dim=128, rope_d_rot=2 * 2048)

# The QKV layer's forward with its filters generated in the kernel from the 2048-wide
# hidden state (the layer input of a ~2B model).
WORKLOADS["gen_qkv_headwise_bf16"] = WORKLOADS["qkv_headwise_bf16"].with_(
    name="gen_qkv_headwise_bf16", gen_hidden=2048, backward=False)

# The short convolutions of linear-RNN hosts at the ~2B scale of the workloads above
# (model width 2048), with per-channel dynamic filters (one channel per filter) and no
# residual (the dynamic convolution takes the place of the host's static one):
# Mamba-2 convolves x, B and C together: expand 2 (4096) + 2 x d_state 128 (one group);
WORKLOADS["mamba2_xbc_headwise_bf16"] = Workload("mamba2_xbc_headwise_bf16", "headwise", B=8, T=4096,
                                                 D=4096 + 2 * 128, W=4, residual=0, dtype="bf16", Hc=1)
# Gated DeltaNet convolves q, k (2048 each) and v (expand 2: 4096).
WORKLOADS["gdn_qkv_headwise_bf16"] = Workload("gdn_qkv_headwise_bf16", "headwise", B=8, T=4096,
                                              D=2048 + 2048 + 4096, W=4, residual=0, dtype="bf16", Hc=1)

# Paths beside the matrix-core and power-of-two head layouts, at the sizes above: the
# R=32 low-rank layer in fp32 (vector-ALU kernels, sums over tokens and channels in
# double), and the QKV layer with 24-channel filter heads (per-head taps at run time,
# dw by whole 8-channel groups).
WORKLOADS["lowrank_f32"] = Workload("lowrank_f32", "lowrank", B=8, T=4096, D=2048, W=4, residual=0,
                                    dtype="f32", R=32, U_std=1.0 / math.sqrt(32 * 4))
WORKLOADS["qkv_headwise24_bf16"] = Workload("qkv_headwise24_bf16", "headwise", B=8, T=4096, D=3 * 2048, W=4,
                                            residual=1, dtype="bf16", Hc=24)

# Seed per workload: a fixed base plus the workload's position in the list above.
BASE_SEED = 20261203
SEEDS = {name: BASE_SEED + i + 1 for i, name in enumerate(WORKLOADS)}


def packed_positions(B: int, T: int, mean_len: float, seed: int) -> np.ndarray:
    """Positions of tokens within packed sequences, [B, T] int32: each row is filled
    with sequences of lengths 1 + Geometric(1/mean_len) (the last one cut at T), and
    pos counts 0, 1, ... from each sequence start."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = np.empty((B, T), np.int32)
    for b in range(B):
        t = 0
        while t < T:
            n = int(min(T - t, rng.geometric(1.0 / max(mean_len, 1.0))))
            pos[b, t:t + n] = np.arange(n, dtype=np.int32)
            t += n
    return pos


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty(a.shape, dtype=np.uint16)
    # chunked to bound temporaries at large sizes
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step]
        flat_o[s:s + step] = ((v + (((v >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_float(a: np.ndarray) -> np.ndarray:
    """Storage array (float32 or bf16 bits) to float64, exactly."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def draw(wl: Workload, seed: int | None = None, need_dy: bool | None = None) -> dict:
    """Draw the inputs of ``wl``: x, then w (headwise) or z and U (lowrank), then dy.

    Arrays are C-contiguous: x, dy [B,T,D]; w [B,T,G,W]; z [B,T,R]; U [R, D*W].
    bf16 tensors are returned as uint16 bit patterns.
    """
    if seed is None:
        seed = SEEDS.get(wl.name, BASE_SEED)
    if need_dy is None:
        need_dy = wl.backward
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"x": _normal(rng, (wl.B, wl.T, wl.D), wl.x_std, wl.dtype)}
    if wl.kind == "headwise":
        out["w"] = _normal(rng, (wl.B, wl.T, wl.G, wl.W), wl.w_std, wl.dtype)
    else:
        out["z"] = _normal(rng, (wl.B, wl.T, wl.R), wl.z_std, wl.dtype)
        out["U"] = _normal(rng, (wl.R, wl.D * wl.W), wl.U_std, wl.dtype)
    if need_dy:
        out["dy"] = _normal(rng, (wl.B, wl.T, wl.D), wl.dy_std, wl.dtype)
    if wl.packed_mean > 0:
        out["pos"] = packed_positions(wl.B, wl.T, wl.packed_mean, seed + 1)
    return out


# ----------------------------------------------------------------------------- decoding

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: B rows (sequences), one new token each, a ring of W-1 inputs per row."""

    name: str
    kind: str            # "headwise" or "lowrank"
    B: int
    D: int
    W: int
    residual: int
    dtype: str
    Hc: int = 0
    R: int = 0
    x_std: float = 1.0
    w_std: float = 0.5
    z_std: float = 1.0
    U_std: float = 0.0
    max_pos: int = 4096  # positions are drawn in [W-1, max_pos): every row has a full ring

    @property
    def G(self) -> int:
        return self.D // self.Hc if self.kind == "headwise" else self.D


# The layers of the training workloads above at generation time, a serving batch of 256 rows.
DECODE_WORKLOADS = {
    "decode_qkv_headwise_bf16": DecodeWorkload("decode_qkv_headwise_bf16", "headwise", B=256, D=3 * 2048, W=4,
                                               residual=1, dtype="bf16", Hc=8),
    "decode_lowrank_bf16": DecodeWorkload("decode_lowrank_bf16", "lowrank", B=256, D=2048, W=4, residual=0,
                                          dtype="bf16", R=32, U_std=1.0 / math.sqrt(32 * 4)),
    "decode_longseq_lowrank_bf16": DecodeWorkload("decode_longseq_lowrank_bf16", "lowrank", B=256, D=4096, W=8,
                                                  residual=0, dtype="bf16", R=64, U_std=1.0 / math.sqrt(64 * 8)),
}
DECODE_SEEDS = {name: BASE_SEED + 101 + i for i, name in enumerate(DECODE_WORKLOADS)}


def draw_decode(wl: DecodeWorkload, seed: int | None = None) -> dict:
    """Inputs of one decode step, in the order x, w (or z, U), state, pos.

    x [B,D]; w [B,G,W]; z [B,R]; U [R,D*W]; state [B,W-1,D] (Gaussian like x: the
    inputs of earlier steps); pos [B] int32 uniform in [W-1, max_pos).
    """
    if seed is None:
        seed = DECODE_SEEDS.get(wl.name, BASE_SEED + 100)
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"x": _normal(rng, (wl.B, wl.D), wl.x_std, wl.dtype)}
    if wl.kind == "headwise":
        out["w"] = _normal(rng, (wl.B, wl.G, wl.W), wl.w_std, wl.dtype)
    else:
        out["z"] = _normal(rng, (wl.B, wl.R), wl.z_std, wl.dtype)
        out["U"] = _normal(rng, (wl.R, wl.D * wl.W), wl.U_std, wl.dtype)
    out["state"] = _normal(rng, (wl.B, wl.W - 1, wl.D), wl.x_std, wl.dtype)
    out["pos"] = rng.integers(wl.W - 1, max(wl.W, wl.max_pos), size=wl.B).astype(np.int32)
    return out


# ----------------------------------------------------------------------------- rotary tables

def rope_table(n_pos: int, head_dim: int, base: float = 10000.0):
    """The usual rotary-embedding cache, float32 [n_pos, head_dim/2] each: cos and sin of
    p * base^(-2i/head_dim) at position p, pair index i (angles in float64, then rounded)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * base ** (-2.0 * i / head_dim)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# ----------------------------------------------------------------------------- generator in the kernel

def draw_gen(wl: Workload, K: int, seed: int | None = None) -> dict:
    """Inputs of the forward with generated filters: x [B,T,D], the hidden state h [B,T,K]
    and the generator weight Wg [G*W, K] ~ N(0, w_std^2 / K), so that the generated filters
    have the spread of the workload's drawn ones."""
    if seed is None:
        seed = SEEDS.get(wl.name, BASE_SEED) + 500
    rng = np.random.Generator(np.random.PCG64(seed))
    return {"x": _normal(rng, (wl.B, wl.T, wl.D), wl.x_std, wl.dtype),
            "h": _normal(rng, (wl.B, wl.T, K), 1.0, wl.dtype),
            "Wg": _normal(rng, (wl.G * wl.W, K), wl.w_std / math.sqrt(K), wl.dtype)}
