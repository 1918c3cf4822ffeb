// Low-rank dynamic short convolution on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// Operation ("Dynamic Short Convolutions Improve Transformers", technical
// summary page, section Metodologia, low-rank factorisation, and the
// fused-kernel section): with the filter of channel c, tap k at step t
//   f[t,c,k] = sum_r z[t,r] U[r, c*W+k],
//   y[t,c]   = residual*x[t,c] + sum_k f[t,c,k] x[t-k,c],
// and, with g[t,c,k] = dy[t,c] x[t-k,c] (chain rule),
//   dx[s,c] = residual*dy[s,c] + sum_k f[s+k,c,k] dy[s+k,c],
//   dz[t,r] = sum_{c,k} g[t,c,k] U[r,c*W+k],
//   dU[r,c*W+k] = sum_t z[t,r] g[t,c,k].
// The three contractions over r, over (c,k) and over t run on
// v_mfma_f32_16x16x32_bf16; f lives only in MFMA accumulators.
//
// Lane layout shared by every kernel here ("step-major"): a wave handles 16
// consecutive steps; lane l holds step t0 + l%16 and 4*QT consecutive
// channels picked by l/16. That is exactly the MFMA accumulator layout when
// the MFMA's M index is a channel and its N index a step, so f comes out of
// the matrix core already lined up with the x, dy, y rows the lane loads.
// Shifts along time (x[t-k], and f*dy moved back by k steps for dx) stay inside
// each 16-lane row and use DPP row shifts, with the rows of the previous (or
// next) 16 steps entering through the rotate-and-merge form.
//
// MFMA 16x16x32 bf16 (checked on the device): lane l supplies A row l%16 and
// B column l%16, eight K values each (the same K slots for A and B), and gets
// C[4*(l/16)+i][l%16] in accumulator i.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace dsc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// DPP controls within each row of 16 lanes.
constexpr int kRowShl = 0x100, kRowShr = 0x110, kRowRor = 0x120;

// Value of lane (i-K) of this 16-lane row; lanes i < K take lane (i-K+16) of `prev`.
template <int K>
__device__ __forceinline__ uint32_t rows_back(uint32_t prev, uint32_t cur) {
  const int wrapped = __builtin_amdgcn_mov_dpp((int)prev, kRowRor + K, 0xf, 0xf, false);
  return (uint32_t)__builtin_amdgcn_update_dpp(wrapped, (int)cur, kRowShr + K, 0xf, 0xf, false);
}
// Value of lane (i+K), zero where i+K >= 16.
template <int K>
__device__ __forceinline__ float lanes_up(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kRowShl + K, 0xf, 0xf, true));
}
// Value of lane (i-K), zero where i < K.
template <int K>
__device__ __forceinline__ float lanes_down(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kRowShr + K, 0xf, 0xf, true));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  u32x4_t q;
  q.x = pack_bf16x2(v[0], v[1]);
  q.y = pack_bf16x2(v[2], v[3]);
  q.z = pack_bf16x2(v[4], v[5]);
  q.w = pack_bf16x2(v[6], v[7]);
  return as_bf16x8(q);
}

// g = dy * x is a product of two bf16 values (16 significant bits): hi + lo, both
// bf16, carry it to within 2^-17 relative. The dz and dU contractions sum
// thousands of such terms, so both parts go through the matrix cores: one bf16
// rounding of g would leave an error of about 1e-3 of the typical magnitude of
// the sum, far above the tolerance for elements near zero.
__device__ __forceinline__ void split_hi_lo(const float* v, bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t h, l;
  uint32_t* hw = reinterpret_cast<uint32_t*>(&h);
  uint32_t* lw = reinterpret_cast<uint32_t*>(&l);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hw[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    lw[i] = pack_bf16x2(v[2 * i] - bf16_lo(hw[i]), v[2 * i + 1] - bf16_hi(hw[i]));
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

__device__ __forceinline__ uint16_t ld_bits(const bf16_t* p) { return p->bits; }

// N dwords (2N bf16 channels) of one row; zero when !ok.
template <int N>
__device__ __forceinline__ void load_row(const bf16_t* p, bool ok, uint32_t (&v)[N]) {
  if constexpr (N == 4) {
    u32x4_t q = ok ? ld_stream<u32x4_t>(p) : u32x4_t{0, 0, 0, 0};
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else if constexpr (N == 8) {
    u32x4_t q0 = ok ? ld_stream<u32x4_t>(p) : u32x4_t{0, 0, 0, 0};
    u32x4_t q1 = ok ? ld_stream<u32x4_t>(p + 8) : u32x4_t{0, 0, 0, 0};
    v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
    v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
  } else {
    static_assert(N == 2, "row width");
    u32x2_t q = ok ? ld_stream<u32x2_t>(p) : u32x2_t{0, 0};
    v[0] = q.x; v[1] = q.y;
  }
}

template <int N>
__device__ __forceinline__ void store_row(bf16_t* p, const float (&v)[2 * N]) {
  if constexpr (N == 2) {
    u32x2_t q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    st_stream<u32x2_t>(p, q);
  } else {
#pragma unroll
    for (int h = 0; h < N / 4; ++h) {
      u32x4_t q;
      q.x = pack_bf16x2(v[8 * h + 0], v[8 * h + 1]);
      q.y = pack_bf16x2(v[8 * h + 2], v[8 * h + 3]);
      q.z = pack_bf16x2(v[8 * h + 4], v[8 * h + 5]);
      q.w = pack_bf16x2(v[8 * h + 6], v[8 * h + 7]);
      st_stream<u32x4_t>(p + 8 * h, q);
    }
  }
}

template <int N>
__device__ __forceinline__ void unpack_row(const uint32_t (&v)[N], float (&f)[2 * N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}

// B operand of the filter contraction: z[row, 32s + 8*(l/16) .. +7]; zero past R or outside [0,T).
template <int KS>
__device__ __forceinline__ void load_z(const bf16_t* zrow, bool row_ok, int R, int g, bf16x8_t (&zb)[KS]) {
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int r0 = 32 * s + 8 * g;
    const u32x4_t q = (row_ok && r0 < R) ? ld_stream<u32x4_t>(zrow + r0) : u32x4_t{0, 0, 0, 0};
    zb[s] = as_bf16x8(q);
  }
}

// A operand of the filter contraction for channel c, tap k: U[32s + 8*(l/16) + j, c*W + k], j < 8.
template <int W>
__device__ __forceinline__ bf16x8_t load_ut(const bf16_t* U, int64_t DW, int64_t c, bool c_ok, int k, int s,
                                            int g, int R) {
  u32x4_t q = {0, 0, 0, 0};
  uint32_t* w = reinterpret_cast<uint32_t*>(&q);
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const int r = 32 * s + 8 * g + j;
    const uint32_t lo = (c_ok && r < R) ? ld_bits(U + (int64_t)r * DW + c * W + k) : 0u;
    const uint32_t hi = (c_ok && r + 1 < R) ? ld_bits(U + (int64_t)(r + 1) * DW + c * W + k) : 0u;
    w[j / 2] = lo | (hi << 16);
  }
  return as_bf16x8(q);
}

struct LowrankArgs {
  const void* x;
  const void* z;
  const void* U;
  const void* dy;
  void* out;         // y (forward) or dx (backward)
  float* dU_part;    // [B * n_split][R][D*W] (backward)
  float* dz_part;    // [n_csplit][B*T][R] (dz kernel)
  int64_t B, T, D;
  int R, residual;
  int n_cblk, n_split;
  int64_t split_len;  // steps per split, a multiple of 32
  // dz kernel
  int n_rtile, n_csplit;
  int64_t csplit_len;  // channels per split, a multiple of 16
};

// ----------------------------------------------------------------------------- forward

// Block: 4 waves over 64*QT channels (wave w: channels cblk*64*QT + w*16*QT ..), all
// walking the steps [ta, tb) of one sequence, 16 at a time. The filter operands
// (U^T, 8 ranks per lane) stay in registers for the whole walk.
template <int W, int KS, int QT>
__global__ __launch_bounds__(256) void lowrank_fwd_mfma_kernel(LowrankArgs a) {
  constexpr int XN = 2 * QT;  // dwords of x per lane per step (4*QT channels)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = lane & 15, g = lane >> 4;
  const uint32_t cblk = blockIdx.x % a.n_cblk;
  const uint32_t rest = blockIdx.x / a.n_cblk;
  const int64_t split = rest % a.n_split, b = rest / a.n_split;
  const int64_t T = a.T, D = a.D, DW = D * W;
  const int R = a.R;
  const int64_t ta = split * a.split_len;
  const int64_t tb = ta + a.split_len < T ? ta + a.split_len : T;
  const int64_t cw0 = (int64_t)cblk * 64 * QT + wave * 16 * QT;
  const int64_t cl = cw0 + 4 * QT * g;  // first of this lane's 4*QT channels
  const bool lane_ok = cl < D;          // D is a multiple of 4*QT: chunks are whole
  const bf16_t* U = static_cast<const bf16_t*>(a.U);
  const bf16_t* zs = static_cast<const bf16_t*>(a.z) + b * T * R;
  const bf16_t* xs = static_cast<const bf16_t*>(a.x) + b * T * D + cl;
  bf16_t* ys = static_cast<bf16_t*>(a.out) + b * T * D + cl;
  const float res = a.residual ? 1.f : 0.f;

  // A operands. Tile q row m is channel cw0 + 4*QT*(m/4) + 4q + m%4, so lane (t, g)
  // receives channels cl + 4q + i (i < 4) from tile q: 4*QT consecutive channels.
  bf16x8_t ua[QT][W][KS];
  {
    const int64_t cA0 = cw0 + 4 * QT * (tl >> 2) + (tl & 3);
#pragma unroll
    for (int q = 0; q < QT; ++q)
#pragma unroll
      for (int k = 0; k < W; ++k)
#pragma unroll
        for (int s = 0; s < KS; ++s) ua[q][k][s] = load_ut<W>(U, DW, cA0 + 4 * q, cA0 + 4 * q < D, k, s, g, R);
  }

  uint32_t xprev[XN], xcur[XN];
  bf16x8_t zcur[KS];
  {
    const int64_t r = ta - 16 + tl;
    load_row<XN>(xs + r * D, lane_ok && r >= 0 && r < T, xprev);
    const int64_t t = ta + tl;
    load_row<XN>(xs + t * D, lane_ok && t < T, xcur);
    load_z<KS>(zs + t * R, t < T, R, g, zcur);
  }
  for (int64_t t0 = ta; t0 < tb; t0 += 16) {
    const int64_t t = t0 + tl;
    // prefetch the next 16 steps
    uint32_t xnext[XN];
    bf16x8_t znext[KS];
    {
      const int64_t tn = t + 16;
      const bool more = t0 + 16 < tb;
      load_row<XN>(xs + tn * D, more && lane_ok && tn < T, xnext);
      load_z<KS>(zs + tn * R, more && tn < T, R, g, znext);
    }
    f32x4_t f[QT][W];
#pragma unroll
    for (int q = 0; q < QT; ++q)
#pragma unroll
      for (int k = 0; k < W; ++k) {
        f[q][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) f[q][k] = mfma_16x16x32(ua[q][k][s], zcur[s], f[q][k]);
      }
    float out[4 * QT], xf[4 * QT];
    unpack_row<XN>(xcur, xf);
#pragma unroll
    for (int q = 0; q < QT; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[4 * q + i] = fmaf(f[q][0][i], xf[4 * q + i], res * xf[4 * q + i]);
    static_for<1, W>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      uint32_t xk[XN];
#pragma unroll
      for (int i = 0; i < XN; ++i) xk[i] = rows_back<k>(xprev[i], xcur[i]);
      float xkf[4 * QT];
      unpack_row<XN>(xk, xkf);
#pragma unroll
      for (int q = 0; q < QT; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[4 * q + i] = fmaf(f[q][k][i], xkf[4 * q + i], out[4 * q + i]);
    });
    if (lane_ok && t < tb) store_row<XN>(ys + t * D, out);
#pragma unroll
    for (int i = 0; i < XN; ++i) {
      xprev[i] = xcur[i];
      xcur[i] = xnext[i];
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) zcur[s] = znext[s];
  }
}

// ----------------------------------------------------------------------------- backward: dx and dU

// LDS row pitch (bf16 elements) of the per-wave transposed staging tiles: 32 steps
// plus padding that spreads consecutive rows over the banks.
constexpr int kStagePitch = 40;

template <int W, int RT>
struct alignas(16) DxdUShared {
  bf16_t g_t[4][2][16 * W][kStagePitch];  // per wave: g[step][column] transposed (hi, lo), column = ch*W + k
  bf16_t z_t[4][16 * RT][kStagePitch];  // per wave: z[step][r] transposed
};

// Block: 4 waves over 64 channels (wave w: channels cblk*64 + 16w .. +15; lane (t, g)
// holds channels +4g .. +4g+3), walking steps [ta, tb) of one sequence.
// dx: f*dy at step t is moved back by k steps (DPP) and summed; the last 16 steps of
//     each block of 16 are completed by the next block, and one extra block past tb
//     completes the end of the range.
// dU: g (as bf16 hi + lo) is staged transposed in LDS with z, 32 steps at a time, so the
//     contraction over steps runs on the matrix cores with the partial sums for the
//     wave's 16*W columns held in accumulators across the whole range.
template <int W, int KS, int RT>
__global__ __launch_bounds__(256) void lowrank_dxdU_kernel(LowrankArgs a) {
  __shared__ DxdUShared<W, RT> sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = lane & 15, g = lane >> 4;
  const uint32_t cblk = blockIdx.x % a.n_cblk;
  const uint32_t rest = blockIdx.x / a.n_cblk;
  const int64_t split = rest % a.n_split, b = rest / a.n_split;
  const int64_t T = a.T, D = a.D, DW = D * W;
  const int R = a.R;
  const int64_t ta = split * a.split_len;
  const int64_t tb = ta + a.split_len < T ? ta + a.split_len : T;
  const int64_t cw0 = (int64_t)cblk * 64 + wave * 16;
  const int64_t cl = cw0 + 4 * g;
  const bool lane_ok = cl < D;  // D is a multiple of 4
  const bf16_t* U = static_cast<const bf16_t*>(a.U);
  const bf16_t* zs = static_cast<const bf16_t*>(a.z) + b * T * R;
  const bf16_t* xs = static_cast<const bf16_t*>(a.x) + b * T * D + cl;
  const bf16_t* dys = static_cast<const bf16_t*>(a.dy) + b * T * D + cl;
  bf16_t* dxs = static_cast<bf16_t*>(a.out) + b * T * D + cl;
  const float res = a.residual ? 1.f : 0.f;
  auto& gT = sh.g_t[wave];
  auto& zT = sh.z_t[wave];

  bf16x8_t ua[W][KS];  // tile row m = channel cw0 + m
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int s = 0; s < KS; ++s) ua[k][s] = load_ut<W>(U, DW, cw0 + tl, cw0 + tl < D, k, s, g, R);

  f32x4_t accU[RT][W];
#pragma unroll
  for (int m = 0; m < RT; ++m)
#pragma unroll
    for (int n = 0; n < W; ++n) accU[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint32_t xprev[2], xcur[2], dycur[2];
  bf16x8_t zcur[KS];
  {
    const int64_t r = ta - 16 + tl;
    load_row<2>(xs + r * D, lane_ok && r >= 0 && r < T, xprev);
    const int64_t t = ta + tl;
    load_row<2>(xs + t * D, lane_ok && t < T, xcur);
    load_row<2>(dys + t * D, lane_ok && t < T, dycur);
    load_z<KS>(zs + t * R, t < T, R, g, zcur);
  }
  float dxc[4] = {0.f, 0.f, 0.f, 0.f};  // pending dx of the previous 16 steps
  int half = 0;                          // which 16-step half of the LDS stage is next
  for (int64_t t0 = ta;; t0 += 16) {
    const bool tail = t0 >= tb;  // the extra block that only completes dx of the last one
    const int64_t t = t0 + tl;
    uint32_t xnext[2], dynext[2];
    bf16x8_t znext[KS];
    {
      const int64_t tn = t + 16;
      const bool more = !tail && tn < T;
      load_row<2>(xs + tn * D, more && lane_ok && t0 + 16 < tb, xnext);
      load_row<2>(dys + tn * D, more && lane_ok, dynext);
      load_z<KS>(zs + tn * R, more, R, g, znext);
    }
    // filters of these 16 steps
    f32x4_t f[W];
#pragma unroll
    for (int k = 0; k < W; ++k) {
      f[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) f[k] = mfma_16x16x32(ua[k][s], zcur[s], f[k]);
    }
    float dyf[4];
    unpack_row<2>(dycur, dyf);
    // dx: p_k = f_k * dy at step t contributes to dx at step t-k
    float cur[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = fmaf(f[0][i], dyf[i], res * dyf[i]);
    static_for<1, W>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = f[k][i] * dyf[i];
        cur[i] += lanes_up<k>(p);         // to step t-k in this block
        dxc[i] += lanes_down<16 - k>(p);  // to step t-k in the previous block
      }
    });
    if (t0 > ta) {
      const int64_t tp = t - 16;
      if (lane_ok && tp < tb) store_row<2>(dxs + tp * D, dxc);
    }
    if (tail) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) dxc[i] = cur[i];

    // g_k = dy * x[t-k] for steps inside [ta, tb); staged transposed with z
    const bool row_in = t < tb;
    float gk[4][W];
    {
      float xf[4];
      unpack_row<2>(xcur, xf);
#pragma unroll
      for (int i = 0; i < 4; ++i) gk[i][0] = row_in ? dyf[i] * xf[i] : 0.f;
    }
    static_for<1, W>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      uint32_t xk[2] = {rows_back<k>(xprev[0], xcur[0]), rows_back<k>(xprev[1], xcur[1])};
      float xkf[4];
      unpack_row<2>(xk, xkf);
#pragma unroll
      for (int i = 0; i < 4; ++i) gk[i][k] = row_in ? dyf[i] * xkf[i] : 0.f;
    });
    const int col_t = 16 * half + tl;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const uint32_t hi = pack_bf16x2(gk[i][k], 0.f) & 0xffffu;
        const uint32_t lo = pack_bf16x2(gk[i][k] - bf16_lo(hi), 0.f) & 0xffffu;
        gT[0][(4 * g + i) * W + k][col_t].bits = (uint16_t)hi;
        gT[1][(4 * g + i) * W + k][col_t].bits = (uint16_t)lo;
      }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t q = __builtin_bit_cast(u32x4_t, zcur[s]);
      const uint32_t zw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 32 * s + 8 * g + j;
        if (r < 16 * RT) zT[r][col_t].bits = (uint16_t)(row_in ? ((j & 1) ? zw[j / 2] >> 16 : zw[j / 2] & 0xffffu) : 0u);
      }
    }
    const bool last = t0 + 16 >= tb;
    if (half == 1 || last) {
      if (half == 0) {  // odd number of 16-step blocks: clear the unused half of both tiles
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int k = 0; k < W; ++k) gT[0][(4 * g + i) * W + k][16 + tl].bits = gT[1][(4 * g + i) * W + k][16 + tl].bits = 0;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 32 * s + 8 * g + j;
            if (r < 16 * RT) zT[r][16 + tl].bits = 0;
          }
      }
      // dU[r, col] += sum over these 32 steps of z[step, r] * g[step, col]
#pragma unroll
      for (int m = 0; m < RT; ++m) {
        const bf16x8_t za = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&zT[16 * m + tl][8 * g]));
#pragma unroll
        for (int n = 0; n < W; ++n) {
          const bf16x8_t ghi = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&gT[0][16 * n + tl][8 * g]));
          const bf16x8_t glo = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&gT[1][16 * n + tl][8 * g]));
          accU[m][n] = mfma_16x16x32(za, ghi, accU[m][n]);
          accU[m][n] = mfma_16x16x32(za, glo, accU[m][n]);
        }
      }
      half = 0;
    } else {
      half = 1;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      xprev[i] = xcur[i];
      xcur[i] = xnext[i];
      dycur[i] = dynext[i];
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) zcur[s] = znext[s];
  }
  // partial dU of this (sequence, split): rows r = 16m + 4g + i, column cw0*W + 16n + tl
  float* dst = a.dU_part + (b * a.n_split + split) * (int64_t)R * DW + cw0 * W;
#pragma unroll
  for (int m = 0; m < RT; ++m)
#pragma unroll
    for (int n = 0; n < W; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * m + 4 * g + i;
        if (r < R && cw0 + (16 * n + tl) / W < D) dst[(int64_t)r * DW + 16 * n + tl] = accU[m][n][i];
      }
}

// ----------------------------------------------------------------------------- backward: dz

// Block: 4 waves, each over MB*16 consecutive steps of one sequence (the block covers
// 64*MB steps), looping over one channel split 16 channels at a time. For every
// 16-channel chunk the U operands (16 ranks x 8 (channel, tap) columns per lane) are
// read once and applied to all MB step blocks; dz accumulates across the chunks.
// Columns within a lane are (channel, tap) pairs ordered ch*WP + k, WP = W rounded up
// to even (the padding tap is zero), so each MFMA takes 8 of the lane's own values.
template <int W, int RT, int MB>
__global__ __launch_bounds__(256) void lowrank_dz_kernel(LowrankArgs a) {
  constexpr int WP = (W + 1) & ~1;
  constexpr int KB = WP / 2;  // 4 channels * WP columns = 8*KB per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = lane & 15, g = lane >> 4;
  const uint32_t rt = blockIdx.x % a.n_rtile;
  const uint32_t rest = blockIdx.x / a.n_rtile;
  const int64_t cs = rest % a.n_csplit, b = rest / a.n_csplit;
  const int64_t T = a.T, D = a.D, DW = D * W;
  const int R = a.R;
  const int64_t tw0 = ((int64_t)rt * 4 + wave) * MB * 16;  // first step of this wave
  const int64_t c_begin = cs * a.csplit_len;
  const int64_t c_end = c_begin + a.csplit_len < D ? c_begin + a.csplit_len : D;
  const bf16_t* U = static_cast<const bf16_t*>(a.U);
  const bf16_t* xs = static_cast<const bf16_t*>(a.x) + b * T * D;
  const bf16_t* dys = static_cast<const bf16_t*>(a.dy) + b * T * D;

  f32x4_t acc[MB][RT];
#pragma unroll
  for (int h = 0; h < MB; ++h)
#pragma unroll
    for (int m = 0; m < RT; ++m) acc[h][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (tw0 < T) {
    for (int64_t c0 = c_begin; c0 < c_end; c0 += 16) {
      const int64_t cl = c0 + 4 * g;
      const bool lane_ok = cl < c_end;
      // U operands: rank 16m + tl, this lane group's columns
      bf16x8_t ud[RT][KB];
#pragma unroll
      for (int m = 0; m < RT; ++m) {
        const int r = 16 * m + tl;
        const bf16_t* urow = U + (int64_t)r * DW + cl * W;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if constexpr (WP == W) {
            const u32x4_t q = (lane_ok && r < R) ? *reinterpret_cast<const u32x4_t*>(urow + 8 * kb) : u32x4_t{0, 0, 0, 0};
            ud[m][kb] = as_bf16x8(q);
          } else {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int col = 8 * kb + j, ch = col / WP, k = col % WP;
              v[j] = (lane_ok && r < R && k < W) ? load1(urow + ch * W + k) : 0.f;
            }
            ud[m][kb] = pack8(v);
          }
        }
      }
      uint32_t xprev[2];
      {
        const int64_t r = tw0 - 16 + tl;
        load_row<2>(xs + r * D + cl, lane_ok && r >= 0 && r < T, xprev);
      }
#pragma unroll
      for (int h = 0; h < MB; ++h) {
        const int64_t t = tw0 + 16 * h + tl;
        const bool ok = lane_ok && t < T;
        uint32_t xcur[2], dyv[2];
        load_row<2>(xs + t * D + cl, ok, xcur);
        load_row<2>(dys + t * D + cl, ok, dyv);
        float dyf[4], gv[4 * WP];
        unpack_row<2>(dyv, dyf);
        {
          float xf[4];
          unpack_row<2>(xcur, xf);
#pragma unroll
          for (int i = 0; i < 4; ++i) gv[i * WP] = dyf[i] * xf[i];
        }
        static_for<1, W>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          uint32_t xk[2] = {rows_back<k>(xprev[0], xcur[0]), rows_back<k>(xprev[1], xcur[1])};
          float xkf[4];
          unpack_row<2>(xk, xkf);
#pragma unroll
          for (int i = 0; i < 4; ++i) gv[i * WP + k] = dyf[i] * xkf[i];
        });
        if constexpr (WP != W) {
#pragma unroll
          for (int i = 0; i < 4; ++i) gv[i * WP + W] = 0.f;
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          bf16x8_t ghi, glo;
          split_hi_lo(gv + 8 * kb, ghi, glo);
#pragma unroll
          for (int m = 0; m < RT; ++m) {
            acc[h][m] = mfma_16x16x32(ud[m][kb], ghi, acc[h][m]);
            acc[h][m] = mfma_16x16x32(ud[m][kb], glo, acc[h][m]);
          }
        }
        xprev[0] = xcur[0];
        xprev[1] = xcur[1];
      }
    }
  }
  // partial dz of this channel split: lane (t, g) holds dz[t, 16m + 4g + i]
  float* dst = a.dz_part + (cs * a.B + b) * T * (int64_t)R;
#pragma unroll
  for (int h = 0; h < MB; ++h) {
    const int64_t t = tw0 + 16 * h + tl;
    if (t >= T) continue;
#pragma unroll
    for (int m = 0; m < RT; ++m) {
      const int r = 16 * m + 4 * g;
      if (r + 3 < R) {
        *reinterpret_cast<float4*>(dst + t * R + r) = make_float4(acc[h][m][0], acc[h][m][1], acc[h][m][2], acc[h][m][3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r + i < R) dst[t * R + r + i] = acc[h][m][i];
      }
    }
  }
}

}  // namespace dsc
