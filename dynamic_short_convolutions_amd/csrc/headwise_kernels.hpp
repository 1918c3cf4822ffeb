// Head-wise tied dynamic short convolution on gfx950: forward and one-pass backward.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", technical
// summary page, section Metodologia: Mecanismo, head-wise tying, residual):
//   y[b,t,c] = residual*x[b,t,c] + sum_{k<W} w[b,t,c/Hc,k] * x[b,t-k,c]
// and its gradients dx, dw (chain rule).
//
// Work decomposition. A thread owns one "channel group" (8 consecutive
// channels: one 16-byte bf16 vector, two float4 for fp32) and walks a run of
// L consecutive steps of one sequence. The W-tap window of past x rows stays
// in registers, so every x, w and dy element is read from HBM once per run,
// plus the W-1 halo rows at the run's edges, which the neighbouring run reads
// at about the same time (cache hits). A wave covers 64 consecutive channel groups (1 KiB of a
// bf16 row) so every access is a fully coalesced 16-byte-per-lane vector
// access. The loop issues the loads of U rows before using any of them so
// each wave keeps U rows of traffic in flight.
//
// Head layouts (Hc = channels per filter):
//   IN_LANE  Hc in {1,2,4,8}:   a group holds P = 8/Hc whole heads;
//   ACROSS   Hc = 8*P, P = 2..64 a power of two: a head spans P lanes, and
//            the backward's per-head sums finish with xor shuffles. Any other
//            multiple of 8 runs as P = 0: the head index computed at run time,
//            y and dx only (dw: headwise_dw_groups_kernel up to Hc = 128);
//   GENERIC  any other Hc:      per-channel head lookup; dw comes from a separate
//            kernel. Where Hc > 8 (P = 2) a group touches at most two heads and
//            keeps their 2W taps and the channel where the second begins (8W
//            expanded taps per step had left the forward 256 registers: 12-channel
//            heads 442 us); else (P = 1) each channel's taps are gathered.
//
// Packed sequences (POS): pos[b,t] is the index of token t within its own
// sequence, and tap k > 0 of step t applies only if k <= pos[b,t]: the window
// keeps its rows, and the taps that would reach into another sequence are
// dropped by selects (not by multiplying with zero, so nothing of a neighbouring
// sequence, not even a NaN, reaches the outputs). Each run loads the positions of
// its steps with its rows; in the backward, a window of positions travels with
// the windows of dy and w.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace dsc {

enum HeadMode { IN_LANE = 0, ACROSS = 1, GENERIC = 2, IN_LANE_TR = 3 };
// IN_LANE_TR (backward only: bf16, one channel per filter, W = 4) is IN_LANE with
// P = 8 whose taps and dw pass through LDS: a lane's 64 bytes of taps per step are
// four 16-byte pieces, 64 bytes apart across the lanes, so one load instruction of
// the plain layout touches 64 lines partly. Here the wave loads its 4 KiB of taps as
// four instructions of 1 KiB each, writes them to a per-wave LDS tile and reads back
// each lane's own 64 bytes (and the reverse for dw). The whole wave takes part, so
// lanes past the last channel stay alive with their loads and stores switched off.

// Number of filter taps a thread holds per row.
template <int W, int MODE, int P>
struct TapCount {
  static constexpr int value = (MODE == IN_LANE || MODE == IN_LANE_TR)
                                  ? P * W
                                  : (MODE == ACROSS ? W : (P == 2 ? 2 * W + 1 : 8 * W));
};

// Orders this wave's LDS accesses for the compiler (one wave's LDS operations run in
// order, so no wait is needed between lanes of the same wave).
__device__ __forceinline__ void hw_wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Load the taps the thread's 8 channels use at one row.
//   wrow: w + row*G*W (start of that row's filters).
template <typename S, int W, int MODE, int P, bool NT = (DSC_LOAD_NT != 0)>
__device__ __forceinline__ void load_taps(const S* wrow, int j, int Hc, int D, int n4,
                                          float (&tp)[TapCount<W, MODE, P>::value]) {
  if constexpr (MODE == IN_LANE) {
    const S* src = wrow + (int64_t)j * P * W;  // heads j*P .. j*P+P-1
    if constexpr (P >= 2) {
      if (n4 == 1) {  // fp32 row ending in a half group: only P/2 heads exist
        float half[P / 2 * W];
        Taps<S, P / 2 * W>::template load<NT>(src, half);
#pragma unroll
        for (int i = 0; i < P / 2 * W; ++i) tp[i] = half[i];
#pragma unroll
        for (int i = P / 2 * W; i < P * W; ++i) tp[i] = 0.f;
        return;
      }
    }
    Taps<S, P * W>::template load<NT>(src, tp);
  } else if constexpr (MODE == ACROSS) {
    // P = 0: Hc = 8P' for any P' (the forward needs only the head of the group)
    const int head = P > 0 ? j / (P > 0 ? P : 1) : 8 * j / Hc;
    Taps<S, W>::template load<NT>(wrow + (int64_t)head * W, tp);
  } else if constexpr (P == 2) {
    // GENERIC with Hc > 8: the group's 8 channels lie in at most two heads; the taps
    // of both (tp[k], tp[W + k]) and, in tp[2W] as integer bits, the index within
    // the group of the first channel of the second head (8 or more: none)
    const int h0 = 8 * j / Hc, c1 = (h0 + 1) * Hc;
    float t0[W], t1[W];
    Taps<S, W>::template load<NT>(wrow + (int64_t)h0 * W, t0);
    if (c1 < 8 * j + 4 * n4) {  // a channel of the group lies in the second head (which then exists)
      Taps<S, W>::template load<NT>(wrow + (int64_t)(h0 + 1) * W, t1);
    } else {
#pragma unroll
      for (int k = 0; k < W; ++k) t1[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < W; ++k) {
      tp[k] = t0[k];
      tp[W + k] = t1[k];
    }
    tp[2 * W] = __int_as_float(c1 - 8 * j);
  } else if (Hc >= 8) {
    // 8 channels touch at most two heads: their taps, then each channel's pick
    const int h0 = 8 * j / Hc, h1 = h0 + 1;
    const int c1 = h1 * Hc;  // first channel of the second head
    float t0[W], t1[W];
    Taps<S, W>::template load<NT>(wrow + (int64_t)h0 * W, t0);
    if (c1 < 8 * j + 4 * n4) {  // a channel of the group lies in the second head (which then exists)
      Taps<S, W>::template load<NT>(wrow + (int64_t)h1 * W, t1);
    } else {
#pragma unroll
      for (int k = 0; k < W; ++k) t1[k] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool second = 8 * j + i >= c1;
#pragma unroll
      for (int k = 0; k < W; ++k) tp[i * W + k] = i < 4 * n4 ? (second ? t1[k] : t0[k]) : 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 8 * j + i;
      if (i < 4 * n4) {
        const S* src = wrow + (int64_t)(c / Hc) * W;
#pragma unroll
        for (int k = 0; k < W; ++k) tp[i * W + k] = load1(src + k);
      } else {
#pragma unroll
        for (int k = 0; k < W; ++k) tp[i * W + k] = 0.f;
      }
    }
  }
}

// Tap k of channel i (0..7 within the group).
template <int W, int MODE, int P>
__device__ __forceinline__ float tap_of(const float (&tp)[TapCount<W, MODE, P>::value], int i, int k) {
  if constexpr (MODE == IN_LANE || MODE == IN_LANE_TR) return tp[(i / (8 / P)) * W + k];
  else if constexpr (MODE == ACROSS) return tp[k];
  else if constexpr (P == 2) return i < __float_as_int(tp[2 * W]) ? tp[k] : tp[W + k];
  else return tp[i * W + k];
}

// ----------------------------------------------------------------------------- rotary embedding

// Rotary embedding of the convolution's output on its first rot_groups channel
// groups (the Q and K heads of a QKV layer: the convolution runs before the
// rotary embedding there, section Metodologia, Posicionamento). In each head of
// hd channels, pair i is the channels (i, i + hd/2), or (2i, 2i+1) when
// interleaved, and (a, b) becomes (a cos - b sin, a sin + b cos) with cos, sin
// read from the caller's tables at [p][i] for the token's position p (RoFormer's
// rotation). The backward applies the transpose (the opposite angle) to dy.
struct RopeArgs {
  const float* cos;  // [n_pos][hd/2]
  const float* sin;  // [n_pos][hd/2]
  int64_t n_pos;
  int64_t rot_groups;  // channel groups (of 8) that are rotated: d_rot / 8
  int hd;              // head size: 16 << k, up to 512
  int interleaved;
};

__device__ __forceinline__ int64_t tr_clamp(int64_t t, int64_t T) { return t < T ? t : T - 1; }

// Rotates the thread's 8 channels of group j at position p (clamped to the table).
// With (i, i + hd/2) pairs the partner channels sit hd/16 lanes away (a head's
// groups are consecutive lanes), so every lane takes part in the exchange,
// rotated or not.
template <bool INV>
__device__ __forceinline__ void rope_group(float (&v)[8], int j, int64_t p, const RopeArgs& r) {
  const bool rot = j < r.rot_groups;
  const int64_t pc = p < 0 ? 0 : (p >= r.n_pos ? r.n_pos - 1 : p);
  const int half = r.hd >> 1;
  const int o = (8 * j) & (r.hd - 1);  // offset of the group in its head
  const float sg = INV ? -1.f : 1.f;
  if (r.interleaved) {
    if (rot) {
      const float4 c = *reinterpret_cast<const float4*>(r.cos + pc * half + (o >> 1));
      const float4 s = *reinterpret_cast<const float4*>(r.sin + pc * half + (o >> 1));
      const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sg * s.x, sg * s.y, sg * s.z, sg * s.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float a = v[2 * m], b = v[2 * m + 1];
        v[2 * m] = a * cc[m] - b * ss[m];
        v[2 * m + 1] = a * ss[m] + b * cc[m];
      }
    }
  } else {
    float other[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) other[m] = __shfl_xor(v[m], half >> 3, 64);
    if (rot) {
      const bool first = o < half;
      const float* cr = r.cos + pc * half + (o & (half - 1));
      const float* sr = r.sin + pc * half + (o & (half - 1));
      const float4 c0 = reinterpret_cast<const float4*>(cr)[0], c1 = reinterpret_cast<const float4*>(cr)[1];
      const float4 s0 = reinterpret_cast<const float4*>(sr)[0], s1 = reinterpret_cast<const float4*>(sr)[1];
      const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      // first half: a' = a cos - b sin; second half: b' = a sin + b cos (own value b)
      const float f = first ? -sg : sg;
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = fmaf(f * ss[m], other[m], v[m] * cc[m]);
    }
  }
}

struct Tiling {
  int cg_log2;   // channel groups per block = 1 << cg_log2 (<= 256)
  int L;         // steps per thread
  int n_cblk;    // channel blocks per row
  int n_ttile;   // step tiles per sequence (each (256 >> cg_log2) * L steps)
  uint32_t nblocks;
};

struct ThreadTile {
  int64_t b, t0, t1;
  int j;
  bool active;
};

// Blocks run in one moving window over the tensors (channel block fastest, then
// step tile, then sequence), which beat giving each XCD its own contiguous part of
// the tensors. Workgroups are dealt to the 8 XCDs round robin; within each window
// of 8 * kXcdSteps step tiles, XCD x takes kXcdSteps consecutive tiles of every
// channel block, so the W-1 halo rows a run reads were mostly fetched by the
// previous run on the same XCD and are found in its L2 (in plain order the
// neighbouring runs sit on different XCDs). On MI355X 3 to 6 tiles per XCD were
// about 2% faster than plain order for the QKV layer, 8 slower again. A last
// partial window keeps the plain order.
#ifndef DSC_HW_XCD_STEPS
#define DSC_HW_XCD_STEPS 4
#endif
constexpr uint32_t kXcdSteps = DSC_HW_XCD_STEPS;
static_assert(kXcdSteps >= 1 && kXcdSteps <= 16, "step tiles per XCD");

__device__ __forceinline__ ThreadTile thread_tile(const Tiling& g, int64_t T, int ngroups) {
  const uint32_t lid = blockIdx.x;
  const uint32_t ncb = (uint32_t)g.n_cblk;
  const uint32_t window = 8u * kXcdSteps * (ncb < (1u << 24) ? ncb : (1u << 24));  // no overflow
  uint32_t cblk, rest;  // rest = step tile counted over the whole batch
  if (ncb < (1u << 24) && lid < g.nblocks / window * window) {
    const uint32_t r = lid % window, xcd = r % 8, k = r / 8;
    rest = lid / window * (8u * kXcdSteps) + xcd * kXcdSteps + k / ncb;
    cblk = k % ncb;
  } else {
    cblk = lid % ncb;
    rest = lid / ncb;
  }
  const uint32_t ttile = rest % g.n_ttile;
  ThreadTile tt;
  tt.b = rest / g.n_ttile;
  const int tid = threadIdx.x;
  const int cg = 1 << g.cg_log2;
  tt.j = (int)cblk * cg + (tid & (cg - 1));
  const int sub = tid >> g.cg_log2;
  const int ts = 256 >> g.cg_log2;
  tt.t0 = ((int64_t)ttile * ts + sub) * g.L;
  tt.t1 = tt.t0 + g.L < T ? tt.t0 + g.L : T;
  tt.active = tt.j < ngroups && tt.t0 < T;
  return tt;
}

// ----------------------------------------------------------------------------- forward

struct FwdArgs {
  const void* x;
  const void* w;
  const int32_t* pos;  // [B, T] with POS
  void* y;
  int64_t T, D, G;
  int Hc, residual, ngroups;
  Tiling g;
  RopeArgs rope;  // with ROPE
};

template <typename S, int W, int MODE, int P, int U, bool POS, bool ROPE>
__global__ __launch_bounds__(256) void headwise_fwd_kernel(FwdArgs a) {
  constexpr int NT = TapCount<W, MODE, P>::value;
  const ThreadTile tt = thread_tile(a.g, a.T, a.ngroups);
  if (!tt.active) return;
  const int n4 = (8 * tt.j + 4 < a.D) ? 2 : 1;
  const int64_t D = a.D, GW = a.G * W;
  const S* xs = static_cast<const S*>(a.x) + tt.b * a.T * D + 8 * tt.j;
  const S* ws = static_cast<const S*>(a.w) + tt.b * a.T * GW;
  S* ys = static_cast<S*>(a.y) + tt.b * a.T * D + 8 * tt.j;
  const int32_t* ps = POS ? a.pos + tt.b * a.T : nullptr;
  const float res = a.residual ? 1.f : 0.f;

  // win[k] = x[t-k] of the thread's 8 channels. Before the first step (t = t0) the
  // window holds the halo as of t0-1: win[k] = x[t0-1-k]; each step shifts it by one.
  float win[W][8];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const int64_t r = tt.t0 - 1 - k;
    if (k < W - 1 && r >= 0) Group8<S>::template load<false>(xs + r * D, win[k], n4);
    else {
#pragma unroll
      for (int i = 0; i < 8; ++i) win[k][i] = 0.f;
    }
  }

  // p: the step's position in its sequence (POS only)
  auto step = [&](int64_t t, const float (&xr)[8], const float (&tp)[NT], int p) {
#pragma unroll
    for (int k = W - 1; k > 0; --k)
#pragma unroll
      for (int i = 0; i < 8; ++i) win[k][i] = win[k - 1][i];
#pragma unroll
    for (int i = 0; i < 8; ++i) win[0][i] = xr[i];
    float out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = res * win[0][i];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const bool on = !POS || k == 0 || k <= p;
        acc = fmaf(on ? tap_of<W, MODE, P>(tp, i, k) : 0.f, on ? win[k][i] : 0.f, acc);
      }
      out[i] = acc;
    }
    if constexpr (ROPE) rope_group<false>(out, tt.j, POS ? (int64_t)p : t, a.rope);
    Group8<S>::store(ys + t * D, out, n4);
  };

#ifndef DSC_FWD_NT
#define DSC_FWD_NT 1
#endif
  constexpr bool kNT = DSC_FWD_NT && W - 1 <= U;
  // One iteration of U steps. Loads of rows read once bypass L2 retention
  // (non-temporal): every w row, and x rows except the run's last W-1, which the
  // next run reads again as its halo.
  auto iter = [&](int64_t t, auto last) {
    constexpr bool Ls = decltype(last)::value;
    float xr[U][8], tp[U][NT];
    int pp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kNT && !(Ls && u >= U - (W - 1))) Group8<S>::template load<true>(xs + (t + u) * D, xr[u], n4);
      else Group8<S>::template load<false>(xs + (t + u) * D, xr[u], n4);
      load_taps<S, W, MODE, P, kNT>(ws + (t + u) * GW, tt.j, a.Hc, (int)D, n4, tp[u]);
      pp[u] = POS ? ps[t + u] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) step(t + u, xr[u], tp[u], pp[u]);
  };
  int64_t t = tt.t0;
  if (t + U <= tt.t1) {
    for (; t + 2 * U <= tt.t1; t += U) iter(t, std::false_type{});
    iter(t, std::true_type{});
    t += U;
  }
  for (; t < tt.t1; ++t) {
    float xr[8], tp[NT];
    Group8<S>::load(xs + t * D, xr, n4);
    load_taps<S, W, MODE, P>(ws + t * GW, tt.j, a.Hc, (int)D, n4, tp);
    step(t, xr, tp, POS ? ps[t] : 0);
  }
}

// ----------------------------------------------------------------------------- backward

struct BwdArgs {
  const void* x;
  const void* w;
  const int32_t* pos;  // [B, T] with POS
  const void* dy;
  void* dx;
  void* dw;
  int64_t T, D, G;
  int Hc, residual, ngroups;
  Tiling g;
  RopeArgs rope;  // with ROPE: dy is rotated back on load
};

// Value of the lane that DPP control CTRL names, within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_lane(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the P lanes of one head (lanes j..j+P-1, P a power of two <= 64), the same
// butterfly in every lane of the head (a + b == b + a, so all of them hold the same
// bits). Within a row of 16 lanes the partners come from DPP moves (quad swaps, then
// the half-row and row mirrors), which stay in the VALU; wider heads use LDS shuffles.
template <int P>
__device__ __forceinline__ float head_sum(float v) {
  if constexpr (P >= 2) v += dpp_lane<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (P >= 4) v += dpp_lane<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (P >= 8) v += dpp_lane<0x141>(v);  // row_half_mirror: the other quad of 8
  if constexpr (P >= 16) v += dpp_lane<0x140>(v); // row_mirror: the other 8 of the row
#pragma unroll
  for (int m = 16; m < P; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <typename S, int W, int MODE, int P, int U, bool POS, bool ROPE>
__global__ __launch_bounds__(256) void headwise_bwd_kernel(BwdArgs a) {
  constexpr int NT = TapCount<W, MODE, P>::value;
  constexpr bool TR = MODE == IN_LANE_TR;
  static_assert(!TR || (W == 4 && P == 8 && sizeof(S) == 2 && !ROPE), "IN_LANE_TR layout");
  const ThreadTile tt = thread_tile(a.g, a.T, a.ngroups);
  // Whole heads are active or inactive together (heads never straddle a
  // sub-tile or the end of the row), so the head-sum shuffles below only ever
  // exchange values between lanes that follow the same path. With TR the wave
  // works while its first group exists (the host launches TR only with waves of 64
  // consecutive groups in one sub-tile); lane_on switches the lane's own accesses.
  if (TR ? ((tt.j & ~63) >= a.ngroups || tt.t0 >= a.T) : !tt.active) return;
  const bool lane_on = !TR || tt.j < a.ngroups;
  const int n4 = (8 * tt.j + 4 < a.D) ? 2 : 1;
  const int64_t T = a.T, D = a.D, GW = a.G * W;
  const S* xs = static_cast<const S*>(a.x) + tt.b * T * D + 8 * tt.j;
  const S* dys = static_cast<const S*>(a.dy) + tt.b * T * D + 8 * tt.j;
  const S* ws = static_cast<const S*>(a.w) + tt.b * T * GW;
  S* dxs = static_cast<S*>(a.dx) + tt.b * T * D + 8 * tt.j;
  S* dws = static_cast<S*>(a.dw) + tt.b * T * GW;
  const int32_t* ps = POS ? a.pos + tt.b * T : nullptr;
  const float res = a.residual ? 1.f : 0.f;

  // TR: the wave's tile of 64 groups x 32 taps (64 bytes per group, its four 16-byte
  // chunks placed at chunk c ^ ((group / 4) % 4) so that the lanes of one access spread
  // over the banks), and this lane's pieces: piece h is bytes 16*l + 1024*h of the
  // wave's 4 KiB of a row, i.e. chunk l % 4 of group l / 4 + 16 * h.
  __shared__ __attribute__((aligned(16))) u32x4_t trtile[TR ? 4 : 1][TR ? 64 * 4 : 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t wgrp = tt.j & ~63;  // the wave's first group
  auto chunk_at = [](int grp, int c) { return grp * 4 + (c ^ ((grp >> 2) & 3)); };
  bool piece_on[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) piece_on[h] = TR && wgrp + lane / 4 + 16 * h < a.ngroups;
  // TR: the wave's 4 KiB of taps of one row as this lane's four pieces
  auto tr_load = [&](const S* wrow, u32x4_t (&pc)[4], auto nt) {
    constexpr bool NTL = decltype(nt)::value;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      pc[h] = piece_on[h] ? ld_stream<u32x4_t, NTL>(wrow + wgrp * 32 + 8 * lane + 512 * h) : u32x4_t{0u, 0u, 0u, 0u};
  };
  // TR: pieces -> this lane's 32 taps
  auto tr_taps = [&](const u32x4_t (&pc)[4], float (&tp)[NT]) {
#pragma unroll
    for (int h = 0; h < 4; ++h) trtile[wv][chunk_at(lane / 4 + 16 * h, lane & 3)] = pc[h];
    hw_wave_lds_sync();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_t q = trtile[wv][chunk_at(lane, c)];
      tp[8 * c + 0] = bf16_lo(q.x); tp[8 * c + 1] = bf16_hi(q.x);
      tp[8 * c + 2] = bf16_lo(q.y); tp[8 * c + 3] = bf16_hi(q.y);
      tp[8 * c + 4] = bf16_lo(q.z); tp[8 * c + 5] = bf16_hi(q.z);
      tp[8 * c + 6] = bf16_lo(q.w); tp[8 * c + 7] = bf16_hi(q.w);
    }
    hw_wave_lds_sync();  // the tile is written again by the next row
  };
  auto gload = [&](const S* p, float (&v)[8], auto nt) {
    constexpr bool NTL = decltype(nt)::value;
    if (lane_on) {
      Group8<S>::template load<NTL>(p, v, n4);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
  };

  float xw[W][8];  // xw[k] = x[t-k]
  // dx is accumulated eagerly: step t adds its tap k term w[t,k]*dy[t] to the running
  // sum of dx[t-k], so a step's taps are used as they arrive and no window of past
  // taps or dy rows is kept. da[i] is the sum of dx[t-i]; the terms reach it in the
  // order residual, tap 0, tap 1, ... as in the definition.
  float da[W][8];
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) xw[k][i] = da[k][i] = 0.f;
  // x halo as of step t0-1 (the first step shifts it into place): xw[k] = x[t0-1-k]
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int64_t r = tt.t0 - 1 - k;
    if (r >= 0) gload(xs + r * D, xw[k], std::false_type{});
  }

  // One step at t: x[t] (if t < t1) enters the window, dy[t] and w[t] (if t < T) add
  // their terms to dx[t-k]; dw(t) is complete if t < t1, and dx(t-W+1) is complete if
  // t-W+1 >= t0 (sums for steps before t0 belong to the previous run and are dropped).
  auto step = [&](int64_t t, const float (&xr)[8], const float (&dyr)[8], const float (&tp)[NT], int p) {
#pragma unroll
    for (int k = W - 1; k > 0; --k) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xw[k][i] = xw[k - 1][i];
        da[k][i] = da[k - 1][i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xw[0][i] = xr[i];
      da[0][i] = res * dyr[i];  // dx[t] starts with its residual term
    }
    // tap k of step t exists (POS: k <= its position); then it reaches back to t-k
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const bool on = !POS || k == 0 || k <= p;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        da[k][i] = fmaf(on ? tap_of<W, MODE, P>(tp, i, k) : 0.f, on ? dyr[i] : 0.f, da[k][i]);
    }
    auto pos_of = [&](int) -> int { return p; };  // step t (dw)

    if (t < tt.t1) {
      if constexpr (TR) {
        // dw[t, c, k] = dy[t, c] * x[t-k, c] for the lane's 8 channels, then through the tile
        u32x4_t own[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t wds[4];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const int i = 2 * c + d / 2, k0 = 2 * (d % 2);  // channel i, taps k0, k0+1
            const float g0 = dyr[i] * xw[k0][i];
            const float g1 = dyr[i] * xw[k0 + 1][i];
            wds[d] = pack_bf16x2((!POS || k0 == 0 || k0 <= pos_of(0)) ? g0 : 0.f,
                                 (!POS || k0 + 1 <= pos_of(0)) ? g1 : 0.f);
          }
          own[c] = u32x4_t{wds[0], wds[1], wds[2], wds[3]};
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) trtile[wv][chunk_at(lane, c)] = own[c];
        hw_wave_lds_sync();
        S* drow = dws + t * GW + wgrp * 32;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const u32x4_t q = trtile[wv][chunk_at(lane / 4 + 16 * h, lane & 3)];
          if (piece_on[h]) st_stream<u32x4_t>(drow + 8 * lane + 512 * h, q);
        }
        hw_wave_lds_sync();
      } else if constexpr (MODE == IN_LANE) {
        constexpr int HC = 8 / P;
        float g[P * W];
#pragma unroll
        for (int h = 0; h < P; ++h)
#pragma unroll
          for (int k = 0; k < W; ++k) {
            float s = 0.f;
#pragma unroll
            for (int i = h * HC; i < (h + 1) * HC; ++i) s = fmaf(dyr[i], xw[k][i], s);
            g[h * W + k] = (!POS || k == 0 || k <= pos_of(0)) ? s : 0.f;
          }
        S* dst = dws + t * GW + (int64_t)tt.j * P * W;
        if constexpr (P >= 2) {
          if (n4 == 1) {
            float half[P / 2 * W];
#pragma unroll
            for (int i = 0; i < P / 2 * W; ++i) half[i] = g[i];
            Taps<S, P / 2 * W>::store(dst, half);
          } else {
            Taps<S, P * W>::store(dst, g);
          }
        } else {
          Taps<S, P * W>::store(dst, g);
        }
      } else if constexpr (MODE == ACROSS && P > 0) {  // (P = 0: dx only, dw by its own kernel)
        float g[W];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          float s = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) s = fmaf(dyr[i], xw[k][i], s);
          s = head_sum<P>(s);
          g[k] = (!POS || k == 0 || k <= pos_of(0)) ? s : 0.f;
        }
        if ((tt.j & (P - 1)) == 0) Taps<S, W>::store(dws + t * GW + (int64_t)(tt.j / P) * W, g);
      }
    }
    const int64_t s = t - (W - 1);
    if (s >= tt.t0 && lane_on) Group8<S>::store(dxs + s * D, da[W - 1], n4);
  };

#ifndef DSC_BWD_NT
#define DSC_BWD_NT 1
#endif
  constexpr bool kNT = DSC_BWD_NT && W - 1 <= U;
  // One iteration of U steps inside the run, where the x, dy and w rows all exist.
  // Rows read once are loaded non-temporal; ordinary loads keep in L2 the rows a
  // neighbouring run reads again: x of the run's last W-1 steps (the next run's
  // left halo) and dy and w of its first W-1 steps (the previous run's right
  // halo). The first and the last iteration of a run are therefore separate
  // instances. The halo loads themselves stay ordinary (non-temporal there
  // measured 6% slower).
  auto iter = [&](int64_t t, auto first, auto last) {
    constexpr bool F = decltype(first)::value, Ls = decltype(last)::value;
    float xr[U][8], dyr[U][8], tp[U][NT];
    u32x4_t pc[TR ? U : 1][4];
    int pp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool x_nt = kNT && !(Ls && u >= U - (W - 1));
      const bool d_nt = kNT && !(F && u < W - 1);
      if (x_nt) gload(xs + (t + u) * D, xr[u], std::true_type{});
      else gload(xs + (t + u) * D, xr[u], std::false_type{});
      if (d_nt) {
        gload(dys + (t + u) * D, dyr[u], std::true_type{});
        if constexpr (TR) tr_load(ws + (t + u) * GW, pc[u], std::true_type{});
        else load_taps<S, W, MODE, P, true>(ws + (t + u) * GW, tt.j, a.Hc, (int)D, n4, tp[u]);
      } else {
        gload(dys + (t + u) * D, dyr[u], std::false_type{});
        if constexpr (TR) tr_load(ws + (t + u) * GW, pc[u], std::false_type{});
        else load_taps<S, W, MODE, P, false>(ws + (t + u) * GW, tt.j, a.Hc, (int)D, n4, tp[u]);
      }
      pp[u] = POS ? ps[t + u] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (ROPE) rope_group<true>(dyr[u], tt.j, POS ? (int64_t)pp[u] : t + u, a.rope);
      if constexpr (TR) tr_taps(pc[u], tp[u]);
      step(t + u, xr[u], dyr[u], tp[u], pp[u]);
    }
  };
  int64_t t = tt.t0;
  const int64_t nit = (tt.t1 - tt.t0) / U;  // whole iterations in the run
  if (nit == 1) {
    iter(t, std::true_type{}, std::true_type{});
    t += U;
  } else if (nit >= 2) {
    iter(t, std::true_type{}, std::false_type{});
    for (t += U; t + 2 * U <= tt.t1; t += U) iter(t, std::false_type{}, std::false_type{});
    iter(t, std::false_type{}, std::true_type{});
    t += U;
  }
  // Leftover steps of a run cut by the end of the sequence (fewer than U).
  for (; t < tt.t1; ++t) {
    float xr[8], dyr[8], tp[NT];
    gload(xs + t * D, xr, std::integral_constant<bool, DSC_LOAD_NT != 0>{});
    gload(dys + t * D, dyr, std::integral_constant<bool, DSC_LOAD_NT != 0>{});
    if constexpr (TR) {
      u32x4_t pc[4];
      tr_load(ws + t * GW, pc, std::integral_constant<bool, DSC_LOAD_NT != 0>{});
      tr_taps(pc, tp);
    } else {
      load_taps<S, W, MODE, P>(ws + t * GW, tt.j, a.Hc, (int)D, n4, tp);
    }
    const int p = POS ? ps[t] : 0;
    if constexpr (ROPE) rope_group<true>(dyr, tt.j, POS ? (int64_t)p : t, a.rope);
    step(t, xr, dyr, tp, p);
  }
  // The right halo: the W-1 steps after the run, whose dy and w rows are all loaded
  // before the first is used (rows past the sequence read its last row and are zeroed).
  if constexpr (W > 1) {
    constexpr int H = W - 1;
    float dyr[H][8], tp[H][NT];
    u32x4_t pc[TR ? H : 1][4];
    int ph[H];
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int64_t tj = tt.t1 + j;
      const int64_t tr = tj < T ? tj : T - 1;
      gload(dys + tr * D, dyr[j], std::false_type{});
      if constexpr (TR) tr_load(ws + tr * GW, pc[j], std::false_type{});
      else load_taps<S, W, MODE, P, false>(ws + tr * GW, tt.j, a.Hc, (int)D, n4, tp[j]);
      ph[j] = POS ? ps[tr] : 0;
    }
    if constexpr (TR) {
#pragma unroll
      for (int j = 0; j < H; ++j) tr_taps(pc[j], tp[j]);
    }
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int64_t tj = tt.t1 + j;
      const bool in = tj < T;
      if constexpr (ROPE) rope_group<true>(dyr[j], tt.j, POS ? (int64_t)ph[j] : tr_clamp(tj, T), a.rope);
#pragma unroll
      for (int i = 0; i < 8; ++i) dyr[j][i] = in ? dyr[j][i] : 0.f;
#pragma unroll
      for (int i = 0; i < NT; ++i) tp[j][i] = in ? tp[j][i] : 0.f;
      float xz[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xz[i] = 0.f;
      step(tj, xz, dyr[j], tp[j], in ? ph[j] : 0);
    }
  }
}

// dw for head layouts the fused kernel does not cover: one thread per (token, head).
struct DwArgs {
  const void* x;
  const int32_t* pos;  // [B, T] or null
  const void* dy;
  void* dw;
  int64_t B, T, D, G;
  int Hc;
};

template <typename S, int W>
__device__ __forceinline__ void headwise_dw_generic_item(const DwArgs& a, int64_t idx) {
  const int64_t h = idx % a.G, row = idx / a.G, t = row % a.T;
  const S* x = static_cast<const S*>(a.x);
  const S* dy = static_cast<const S*>(a.dy) + row * a.D + h * a.Hc;
  float g[W];
  const int p = a.pos ? a.pos[row] : W;
  if (a.Hc % 8 == 0) {
    // whole groups of 8 channels: vector loads of dy once and of each x row, the
    // products summed in the same channel order as below
#pragma unroll
    for (int k = 0; k < W; ++k) g[k] = 0.f;
    for (int q = 0; q < a.Hc; q += 8) {
      float dv[8];
      Group8<S>::load(dy + q, dv, 2);
#pragma unroll
      for (int k = 0; k < W; ++k) {
        if (t - k >= 0 && (k == 0 || k <= p)) {
          float xv[8];
          Group8<S>::load(x + (row - k) * a.D + h * a.Hc + q, xv, 2);
#pragma unroll
          for (int i = 0; i < 8; ++i) g[k] = fmaf(dv[i], xv[i], g[k]);
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < W; ++k) {
      float s = 0.f;
      if (t - k >= 0 && (k == 0 || k <= p)) {
        const S* xr = x + (row - k) * a.D + h * a.Hc;
        for (int i = 0; i < a.Hc; ++i) s = fmaf(load1(dy + i), load1(xr + i), s);
      }
      g[k] = s;
    }
  }
  S* dst = static_cast<S*>(a.dw) + idx * W;
#pragma unroll
  for (int k = 0; k < W; ++k) store1(dst + k, g[k]);
}

template <typename S, int W>
__global__ __launch_bounds__(256) void headwise_dw_generic_kernel(DwArgs a) {
  // one (step, head) item per thread, striding over the capped grid
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < a.B * a.T * a.G;
       idx += (int64_t)gridDim.x * blockDim.x)
    headwise_dw_generic_item<S, W>(a, idx);
}

// dw for heads of GC*P channels that the fused kernel leaves to a kernel of its own
// (GC = 8: P = 3, 5, 6, 7, 9 .. 16; GC = 4: head sizes 12, 20, .. 60, multiples of 4
// but not of 8): a block of 64P threads takes 64 heads of one token per item; thread i
// forms the W partial sums of channel group i (GC channels: one 16-byte load, or 8 bytes
// in bf16 with GC = 4, of dy and of each of the W x rows), and thread h < 64 adds the P
// partials of head h in group order. (One thread per (token, head) read the head's
// channels per row at a stride of the head size across the lanes: 740 us of the 1.0 ms
// backward at the QKV layer with 24-channel heads, 1,259 us of 1.55 ms with 12-channel
// heads.)
template <typename S, int W, int GC>
__global__ __launch_bounds__(1024) void headwise_dw_groups_kernel(DwArgs a) {
  static_assert(GC == 8 || GC == 4, "channels per group");
  extern __shared__ float dw_part[];  // [64P][W]
  const int P = a.Hc / GC;
  const int64_t nhb = (a.G + 63) / 64;  // blocks of 64 heads per token
  const int64_t items = a.B * a.T * nhb;
  const S* x = static_cast<const S*>(a.x);
  const S* dy = static_cast<const S*>(a.dy);
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {  // uniform over the block
    const int64_t row = it / nhb, hb = it % nhb, t = row % a.T;
    const int p = a.pos ? a.pos[row] : W;
    const int64_t grp = hb * 64 * P + threadIdx.x;  // this thread's channel group
    float g[W];
#pragma unroll
    for (int k = 0; k < W; ++k) g[k] = 0.f;
    // GC channels at q (16-byte aligned with GC = 8; with GC = 4, 8- or 16-byte aligned
    // as the head size and D are multiples of 4)
    auto load_grp = [](const S* q, float (&v)[GC]) {
      if constexpr (GC == 8) Group8<S>::load(q, v, 2);
      else Taps<S, GC>::template load<false>(q, v);
    };
    if (GC * grp < a.D) {
      float dv[GC];
      load_grp(dy + row * a.D + GC * grp, dv);
#pragma unroll
      for (int k = 0; k < W; ++k) {
        if (t - k >= 0 && (k == 0 || k <= p)) {
          float xv[GC];
          load_grp(x + (row - k) * a.D + GC * grp, xv);
#pragma unroll
          for (int i = 0; i < GC; ++i) g[k] = fmaf(dv[i], xv[i], g[k]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < W; ++k) dw_part[threadIdx.x * W + k] = g[k];
    __syncthreads();
    const int64_t h = hb * 64 + threadIdx.x;
    if (threadIdx.x < 64 && h < a.G) {
      float sum[W];
#pragma unroll
      for (int k = 0; k < W; ++k) sum[k] = dw_part[threadIdx.x * P * W + k];
      for (int q = 1; q < P; ++q)
#pragma unroll
        for (int k = 0; k < W; ++k) sum[k] += dw_part[(threadIdx.x * P + q) * W + k];
      S* dst = static_cast<S*>(a.dw) + (row * a.G + h) * W;
#pragma unroll
      for (int k = 0; k < W; ++k) store1(dst + k, sum[k]);
    }
    __syncthreads();  // dw_part is written again for the next item
  }
}

// ----------------------------------------------------------------------------- launch shape
inline int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}

// Blocks of 256 threads: `cg` channel groups (a power of two, at most 256) times
// 256/cg runs of L steps. L doubles if the grid would reach 2^32 work-items.
inline Tiling make_tiling(int64_t B, int64_t T, int ngroups, int L) {
  Tiling g;
  int cg = 1;
  while (cg < ngroups && cg < 256) cg <<= 1;
  g.cg_log2 = ilog2(cg);
  const int64_t ts = 256 / cg;
  g.n_cblk = (ngroups + cg - 1) / cg;
  int64_t n_ttile, nblocks;
  for (;;) {
    n_ttile = (T + ts * L - 1) / (ts * L);
    nblocks = (int64_t)g.n_cblk * n_ttile * B;
    if (nblocks * 256 <= 0xffffffffLL) break;  // a dispatch counts its work-items in 32 bits
    L *= 2;
  }
  g.L = L;
  g.n_ttile = (int)n_ttile;
  g.nblocks = (uint32_t)nblocks;
  return g;
}

struct HeadLayout {
  int mode, p;
};

inline HeadLayout head_layout(int Hc) {
  if (Hc == 1 || Hc == 2 || Hc == 4 || Hc == 8) return {IN_LANE, 8 / Hc};
  if (Hc % 8 == 0) {
    const int p = Hc / 8;
    if ((p & (p - 1)) == 0 && p <= 64) return {ACROSS, p};
  }
  return {GENERIC, 1};
}

}  // namespace dsc
