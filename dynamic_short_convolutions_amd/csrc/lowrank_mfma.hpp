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
//
// Packed sequences (POS): pos[b,t], the index of token t within its own
// sequence, is loaded per lane with the step's rows; tap k > 0 of step t exists
// only if k <= pos[b,t]. A missing tap is dropped by a select at step t, the
// lane that owns it: the shifted x (forward, g), or the product f_k * dy before
// it is moved back k steps (dx). Nothing of a neighbouring sequence reaches an
// output, not even a NaN.
#pragma once

#include <type_traits>

#include "buffer.hpp"
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

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane
// 4r+q names row r, columns 4q..4q+3 of a row-major tile of 16-bit values, and
// lane j receives column j of those 4 rows (4 values, the first row lowest).
__device__ __forceinline__ uint2 lds_read_tr(const bf16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Eight K slots of an MFMA operand from two transposing reads: column j of rows
// r0 .. r0+3 and r0+4 .. r0+7 of a row-major tile with `pitch` elements per row,
// where `p` is the address lane 4r+q of the group names for the first read.
__device__ __forceinline__ bf16x8_t lds_read_tr8(const bf16_t* p, int pitch) {
  const uint2 a = lds_read_tr(p), b = lds_read_tr(p + 4 * pitch);
  return as_bf16x8(u32x4_t{a.x, a.y, b.x, b.y});
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

// N dwords (2N bf16 channels) of one row at byte offset `off` of buffer `b`
// (kOutOfRange reads zeros). With N = 8 the two 16-byte halves lie HS bytes apart.
template <int N, int HS = 16>
__device__ __forceinline__ void load_row(buf_t b, uint32_t off, uint32_t (&v)[N]) {
  if constexpr (N == 4) {
    const u32x4_t q = buf_load16(b, off);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else if constexpr (N == 8) {
    const u32x4_t q0 = buf_load16(b, off);
    const u32x4_t q1 = buf_load16(b, off == kOutOfRange ? off : off + HS);
    v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
    v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
  } else {
    static_assert(N == 2, "row width");
    const u32x2_t q = buf_load8(b, off);
    v[0] = q.x; v[1] = q.y;
  }
}

// N dwords (2N bf16 channels) of one row, rounded to nearest-even, stored at byte
// offset `off` of buffer `b` (kOutOfRange: dropped); 16-byte pieces HS bytes apart.
template <int N, bool NT, int HS = 16>
__device__ __forceinline__ void store_row(buf_t b, uint32_t off, const float (&v)[2 * N]) {
  if constexpr (N == 2) {
    u32x2_t q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    buf_store8<NT>(b, off, q);
  } else {
#pragma unroll
    for (int h = 0; h < N / 4; ++h) {
      u32x4_t q;
      q.x = pack_bf16x2(v[8 * h + 0], v[8 * h + 1]);
      q.y = pack_bf16x2(v[8 * h + 2], v[8 * h + 3]);
      q.z = pack_bf16x2(v[8 * h + 4], v[8 * h + 5]);
      q.w = pack_bf16x2(v[8 * h + 6], v[8 * h + 7]);
      buf_store16<NT>(b, off == kOutOfRange ? off : off + HS * h, q);
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

// B operand of the filter contraction: z[t, 32s + 8*(l/16) .. +7] of one sequence's
// z (buffer zb); zero past R or when !ok.
template <int KS>
__device__ __forceinline__ void load_z(buf_t zb, int t, bool ok, int R, int g, bf16x8_t (&zv)[KS]) {
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int r0 = 32 * s + 8 * g;
    const uint32_t off = (uint32_t)(t * R + r0) * 2u;
    zv[s] = as_bf16x8(buf_load16(zb, (ok & (r0 < R)) ? off : kOutOfRange));
  }
}

// A operand of the filter contraction for channel c, tap k: U[32s + 8*(l/16) + j, c*W + k], j < 8.
template <int W>
__device__ __forceinline__ bf16x8_t load_ut(buf_t ub, int64_t DW, int64_t c, bool c_ok, int k, int s, int g,
                                            int R) {
  u32x4_t q;
  uint32_t* w = reinterpret_cast<uint32_t*>(&q);
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const int r = 32 * s + 8 * g + j;
    const uint32_t o0 = (c_ok && r < R) ? (uint32_t)(((int64_t)r * DW + c * W + k) * 2) : kOutOfRange;
    const uint32_t o1 = (c_ok && r + 1 < R) ? (uint32_t)(((int64_t)(r + 1) * DW + c * W + k) * 2) : kOutOfRange;
    w[j / 2] = (uint32_t)buf_load2(ub, o0) | ((uint32_t)buf_load2(ub, o1) << 16);
  }
  return as_bf16x8(q);
}

// Position of step t within its packed sequence, through a resource over one
// row's positions (out of range: 0, i.e. tap 0 only).
__device__ __forceinline__ int load_pos(buf_t pb, int t) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(pb, t >= 0 ? (uint32_t)t * 4u : kOutOfRange, 0, 0);
}

struct LowrankArgs {
  const void* x;
  const void* z;
  const void* U;
  const int32_t* pos;  // [B, T] with POS
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

// Orders this wave's LDS accesses for the compiler: writes of one lane read by
// other lanes of the same wave (LDS executes one wave's accesses in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// Block: 4 waves over 64*QT channels (wave w: channels cblk*64*QT + w*16*QT ..), all
// walking the steps [ta, tb) of one sequence, 16 at a time. The filter operands
// (U^T, 8 ranks per lane) stay in registers for the whole walk. The x and z rows
// of the next PF blocks of 16 steps are in flight in a ring of registers indexed
// at compile time (the loop is unrolled PF times), so no wait is forced early.
template <int W, int KS, int QT, int PF, bool POS>
__global__ __launch_bounds__(256) void lowrank_fwd_mfma_kernel(LowrankArgs a) {
  constexpr int XN = 2 * QT;  // dwords of x per lane per step (4*QT channels)
  // non-temporal y stores where the filter work is light and rows are written fast
  constexpr bool kStreamOut = W * KS <= 4;
  // With four tiles a wave owns 64 channels (one 128-byte line) of each step, and a
  // lane's 16 channels are two runs of 8, 32 channels apart: one 16-byte access of
  // the wave then covers a contiguous half line of each row (interleaved 16-byte
  // pieces left every 32-byte piece half written by each of two stores).
  constexpr int HS = QT == 4 ? 64 : 16;  // bytes between a lane's two 16-byte pieces
  // With four tiles the y rows also leave through LDS: the wave's 16 steps x 64
  // channels are written to a per-wave tile and read back so that 8 lanes hold one
  // step's whole 128-byte line, and each store instruction writes 8 full lines (a
  // lane's own pieces covered 16 rows by half lines, and the forward spent more time
  // on its y stores than on all the rest: 89 us with them, 38 without).
  constexpr bool kRowStore = QT == 4;
  constexpr int kYPitch = 64 + 8;  // bf16 per staged row: 64 channels and 16 bytes of padding
  __shared__ __attribute__((aligned(16))) bf16_t ystage[kRowStore ? 4 : 1][16][kRowStore ? kYPitch : 8];
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
  // first of this lane's 4*QT channels (QT = 4: of its first run of 8)
  const int64_t cl = QT == 4 ? cw0 + 8 * g : cw0 + 4 * QT * g;
  // D is a multiple of 4*QT (of 64 with QT = 4): a lane's channels are all valid or none
  const bool lane_ok = cl < D;
  // x, z and y are addressed through resources that end at row tb of this sequence:
  // rows past it read zero (stores are dropped) without a compare. Every per-sequence
  // range is below 2 GiB (checked by the launch plan), so offsets are 32-bit, and lanes
  // past D start at kOutOfRange, beyond every resource.
  const buf_t xb = make_buf(static_cast<const bf16_t*>(a.x) + b * T * D, (uint64_t)(tb * D * 2));
  const buf_t zb = make_buf(static_cast<const bf16_t*>(a.z) + b * T * R, (uint64_t)(tb * R * 2));
  const buf_t ub = make_buf(a.U, (uint64_t)(R * DW * 2));
  const buf_t yb = make_buf(static_cast<bf16_t*>(a.out) + b * T * D, (uint64_t)(tb * D * 2));
  const buf_t pb = make_buf(POS ? a.pos + b * T : nullptr, POS ? (uint64_t)(tb * 4) : 0);
  const float res = a.residual ? 1.f : 0.f;
  const uint32_t row_bytes = (uint32_t)(D * 2);
  const uint32_t lane_base = lane_ok ? (uint32_t)(cl * 2) : kOutOfRange;
  auto x_at = [&](int t) -> uint32_t { return (uint32_t)t * row_bytes + lane_base; };  // t >= 0

  // A operands. Tile q row m is channel cw0 + 4*QT*(m/4) + 4q + m%4, so lane (t, g)
  // receives channels cl + 4q + i (i < 4) from tile q: 4*QT consecutive channels.
  // With QT = 4, tiles 2 and 3 hold the run 32 channels on: channel
  // cw0 + 32*(q/2) + 8*(m/4) + 4*(q%2) + m%4.
  bf16x8_t ua[QT][W][KS];
  {
    const int64_t cA0 = QT == 4 ? cw0 + 8 * (tl >> 2) + (tl & 3) : cw0 + 4 * QT * (tl >> 2) + (tl & 3);
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      const int64_t c = QT == 4 ? cA0 + 32 * (q >> 1) + 4 * (q & 1) : cA0 + 4 * q;
#pragma unroll
      for (int k = 0; k < W; ++k)
#pragma unroll
        for (int s = 0; s < KS; ++s) ua[q][k][s] = load_ut<W>(ub, DW, c, c < D, k, s, g, R);
    }
  }

  // Ring of PF slots: slot s % PF holds the x and z rows of step-block s. x of block s is
  // loaded while block s-PF+1 is computed (it has to outlive one more block as the
  // previous block of s+1); z of block s while block s-PF is computed. Slots are only
  // written by loads and read by the computation, never copied, so the waits for a
  // slot fall just before its use.
  const int nsteps = (int)((tb - ta + 15) / 16);
  const int t0 = (int)ta + tl;
  uint32_t xr[PF][XN];
  bf16x8_t zr[PF][KS];
  int pr[PF];  // positions of block s in slot s % PF, with its z (POS)
  load_row<XN, HS>(xb, t0 >= 16 ? x_at(t0 - 16) : kOutOfRange, xr[PF - 1]);  // block -1: the halo
#pragma unroll
  for (int j = 0; j < PF - 1; ++j) load_row<XN, HS>(xb, x_at(t0 + 16 * j), xr[j]);
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    load_z<KS>(zb, t0 + 16 * j, true, R, g, zr[j]);
    pr[j] = POS ? load_pos(pb, t0 + 16 * j) : 0;
  }
  // Drain the prologue once, so the wait counts at the loop head need only hold for
  // the ring refills (otherwise they drain the whole ring at every pass).
  __builtin_amdgcn_s_waitcnt(0);
  // The loop runs a whole number of rings: steps past the range read zeros (out-of-range
  // loads) and store nothing, which keeps every slot's refill unconditional.
  for (int s0 = 0; s0 < nsteps; s0 += PF) {
    static_for<0, PF>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int jp = (j + PF - 1) % PF;  // slot of the previous block
      const int t = t0 + 16 * (s0 + j);
      f32x4_t f[QT][W];
#pragma unroll
      for (int q = 0; q < QT; ++q)
#pragma unroll
        for (int k = 0; k < W; ++k) {
          // the residual rides on tap 0's accumulator: (f_0 + residual) * x
          f[q][k] = k == 0 ? f32x4_t{res, res, res, res} : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) f[q][k] = mfma_16x16x32(ua[q][k][s], zr[j][s], f[q][k]);
        }
      float out[4 * QT], xf[4 * QT];
      unpack_row<XN>(xr[j], xf);
#pragma unroll
      for (int q = 0; q < QT; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[4 * q + i] = f[q][0][i] * xf[4 * q + i];
      static_for<1, W>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const bool on = !POS || k <= pr[j];
        uint32_t xk[XN];
#pragma unroll
        for (int i = 0; i < XN; ++i) {
          // the row shift runs in every lane (a DPP move reads its neighbours), then the select
          const uint32_t v = rows_back<k>(xr[jp][i], xr[j][i]);
          xk[i] = on ? v : 0u;
        }
        float xkf[4 * QT];
        unpack_row<XN>(xk, xkf);
#pragma unroll
        for (int q = 0; q < QT; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) out[4 * q + i] = fmaf(f[q][k][i], xkf[4 * q + i], out[4 * q + i]);
      });
      if constexpr (kRowStore) {
        bf16_t* rowp = &ystage[wave][tl][0];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4_t q;
          q.x = pack_bf16x2(out[8 * h + 0], out[8 * h + 1]);
          q.y = pack_bf16x2(out[8 * h + 2], out[8 * h + 3]);
          q.z = pack_bf16x2(out[8 * h + 4], out[8 * h + 5]);
          q.w = pack_bf16x2(out[8 * h + 6], out[8 * h + 7]);
          *reinterpret_cast<u32x4_t*>(rowp + 32 * h + 8 * g) = q;  // channels 32h + 8g ..
        }
        wave_lds_sync();
        const int tbase = (int)ta + 16 * (s0 + j);  // step of row 0 of this block
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 8 * h + (lane >> 3), c8 = lane & 7;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&ystage[wave][r][8 * c8]);
          buf_store16<kStreamOut>(yb, cw0 < D ? (uint32_t)(tbase + r) * row_bytes + (uint32_t)((cw0 + 8 * c8) * 2)
                                             : kOutOfRange, v);
        }
        wave_lds_sync();  // the tile is written again by the next block
      } else {
        store_row<XN, kStreamOut, HS>(yb, x_at(t), out);
      }
      // refill: x of block s0+j+PF-1 into the previous block's slot, z of block s0+j+PF into this one
      load_row<XN, HS>(xb, x_at(t + 16 * (PF - 1)), xr[jp]);
      load_z<KS>(zb, t + 16 * PF, true, R, g, zr[j]);
      if constexpr (POS) pr[j] = load_pos(pb, t + 16 * PF);
    });
  }
}

// Forward with time in the lane (W <= 4, W*KS <= 4, D a multiple of 64). The filter
// contraction runs with M = step, N = channel, K = rank: A is z as its rows are
// loaded, B the U operands, and lane (G, j) = (lane/16, lane%16) receives the
// filters of steps 4G .. 4G+3 of channel j of each 16-channel tile. The x rows a
// wave needs (16 steps by its 64 channels, and the 4 steps before them) are
// written to a per-wave LDS ring and read back with transposing reads that hand
// lane j 4 consecutive steps of channel j, so x[t-k] for its four steps are the
// lane's own registers: no lane shifts, one unpack per value, and each output is
// one multiply and W-1 fused multiply-adds (tap 0 carries the residual, as in
// the step-major kernel). The y values go to a per-wave LDS tile and leave by
// whole 128-byte lines, 8 lanes per step.
// Block: 4 waves over 256 channels (wave w: channels cblk*256 + 64w ..) walking the
// steps [ta, tb) of one sequence, 16 at a time, with the x and z rows of the next PF
// blocks in flight in registers (x: lane i holds 16-byte piece i%8 of rows i/8 and
// 8 + i/8, i.e. whole lines).
namespace fwd_tl {
constexpr int kXPitch = 64;      // bf16 per staged x row (128 bytes, pieces swizzled by row)
constexpr int kYPitch = 64 + 8;  // bf16 per staged y row: 64 channels and 16 bytes of padding
// element offset of channel c (0..63) of row r in a staged x slot: 16-byte piece c/8 of
// row r sits at piece position (c/8) ^ (r%8), so that the four rows of a transposing
// read fall on different banks
__device__ __forceinline__ constexpr int xs_at(int r, int c) { return r * kXPitch + 8 * (((c >> 3) ^ r) & 7) + (c & 7); }
}  // namespace fwd_tl

template <int W, int KS, int PF, bool POS>
__global__ __launch_bounds__(256) void lowrank_fwd_tl_kernel(LowrankArgs a) {
  using namespace fwd_tl;
  static_assert(W <= 4 && W * KS <= 4, "taps beyond the four steps staged before a lane's own");
  constexpr int QT = 4;
  // per wave: two 16-step slots of x rows (block s in slot s % 2; rows 12..15 of the
  // other slot are the 4 steps before block s) and the y tile of one block
  __shared__ __attribute__((aligned(16))) bf16_t xs[4][2][16 * kXPitch];
  __shared__ __attribute__((aligned(16))) bf16_t ys[4][16][kYPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, G = lane >> 4;
  const uint32_t cblk = blockIdx.x % a.n_cblk;
  const uint32_t rest = blockIdx.x / a.n_cblk;
  const int64_t split = rest % a.n_split, b = rest / a.n_split;
  const int64_t T = a.T, D = a.D, DW = D * W;
  const int R = a.R;
  const int64_t ta = split * a.split_len;
  const int64_t tb = ta + a.split_len < T ? ta + a.split_len : T;
  const int64_t cw0 = (int64_t)cblk * 256 + wave * 64;
  const bool wave_ok = cw0 < D;  // D is a multiple of 64: a wave's channels are all valid or none
  const buf_t xb = make_buf(static_cast<const bf16_t*>(a.x) + b * T * D, (uint64_t)(tb * D * 2));
  const buf_t zb = make_buf(static_cast<const bf16_t*>(a.z) + b * T * R, (uint64_t)(tb * R * 2));
  const buf_t ub = make_buf(a.U, (uint64_t)(R * DW * 2));
  const buf_t yb = make_buf(static_cast<bf16_t*>(a.out) + b * T * D, (uint64_t)(tb * D * 2));
  const buf_t pb = make_buf(POS ? a.pos + b * T : nullptr, POS ? (uint64_t)(tb * 4) : 0);
  const float res = a.residual ? 1.f : 0.f;
  const uint32_t row_bytes = (uint32_t)(D * 2);
  // lane i's piece of the wave's 128 bytes in rows i/8 and 8 + i/8 of a block
  const int lr = lane >> 3, lp = lane & 7;
  const uint32_t piece_base = wave_ok ? (uint32_t)(cw0 * 2 + 16 * lp) : kOutOfRange;
  auto x_at = [&](int t) -> uint32_t { return (uint32_t)t * row_bytes + piece_base; };  // t >= 0

  // B operands: U[32s + 8G + jj, c*W + k] for channel c = cw0 + 16q + j
  bf16x8_t ub_op[QT][W][KS];
#pragma unroll
  for (int q = 0; q < QT; ++q) {
    const int64_t c = cw0 + 16 * q + j;
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
      for (int s = 0; s < KS; ++s) ub_op[q][k][s] = load_ut<W>(ub, DW, c, c < D, k, s, G, R);
  }

  const int nsteps = (int)((tb - ta + 15) / 16);
  const int tblk0 = (int)ta;
  // rings: x pieces of block s (rows lr and 8 + lr), z rows (A operand: step j), and
  // positions of steps 4G .. 4G+3 (POS), all in slot s % PF
  u32x4_t xr[PF][2];
  bf16x8_t zr[PF][KS];
  u32x4_t pr[PF];
  auto load_x = [&](int blk, u32x4_t (&v)[2]) {  // blk >= -1; rows before the sequence read zero
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = tblk0 + 16 * blk + 8 * h + lr;
      v[h] = buf_load16(xb, t >= 0 ? x_at(t) : kOutOfRange);
    }
  };
  auto load_zp = [&](int blk, int slot) {
    load_z<KS>(zb, tblk0 + 16 * blk + j, true, R, G, zr[slot]);
    if constexpr (POS) {
      // one dword each: a step past the range reads 0 without affecting the others
      const int t = tblk0 + 16 * blk + 4 * G;
      pr[slot] = u32x4_t{(uint32_t)load_pos(pb, t), (uint32_t)load_pos(pb, t + 1), (uint32_t)load_pos(pb, t + 2),
                         (uint32_t)load_pos(pb, t + 3)};
    }
  };
  auto stage_x = [&](int slot, const u32x4_t (&v)[2]) {
    bf16_t* base = &xs[wave][slot][0];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<u32x4_t*>(base + xs_at(8 * h + lr, 8 * lp)) = v[h];
  };
  {
    // block -1 (the 4 steps before the range; zeros at the sequence start) into slot 1
    u32x4_t h0[2];
    load_x(-1, h0);
    __builtin_amdgcn_s_waitcnt(0);
    stage_x(1, h0);
  }
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    load_x(i, xr[i]);
    load_zp(i, i);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const int r4 = j >> 2, q4 = j & 3;
  for (int s0 = 0; s0 < nsteps; s0 += PF) {
    static_for<0, PF>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int blk = s0 + i;
      const int slot = blk & 1;
      stage_x(slot, xr[i]);
      wave_lds_sync();
      // steps 4G-4 .. 4G+3 of channel 16q + j; rows before the block come from the
      // other slot's last 4 rows
      uint32_t xv[QT][4];
      {
        const bf16_t* cur = &xs[wave][slot][0];
        const bf16_t* prv = &xs[wave][slot ^ 1][0];
        const int rlo = 4 * G - 4 + r4, rhi = 4 * G + r4;
        const bf16_t* plo = rlo < 0 ? prv : cur;
        const int rl = rlo < 0 ? rlo + 16 : rlo;
#pragma unroll
        for (int q = 0; q < QT; ++q) {
          const uint2 lo = lds_read_tr(plo + xs_at(rl, 16 * q + 4 * q4));
          const uint2 hi = lds_read_tr(cur + xs_at(rhi, 16 * q + 4 * q4));
          xv[q][0] = lo.x; xv[q][1] = lo.y; xv[q][2] = hi.x; xv[q][3] = hi.y;
        }
      }
      f32x4_t f[QT][W];
#pragma unroll
      for (int q = 0; q < QT; ++q)
#pragma unroll
        for (int k = 0; k < W; ++k) {
          f[q][k] = k == 0 ? f32x4_t{res, res, res, res} : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) f[q][k] = mfma_16x16x32(zr[i][s], ub_op[q][k][s], f[q][k]);
        }
      int pos4[4];
      if constexpr (POS) {
        pos4[0] = (int)pr[i].x; pos4[1] = (int)pr[i].y; pos4[2] = (int)pr[i].z; pos4[3] = (int)pr[i].w;
      }
#pragma unroll
      for (int q = 0; q < QT; ++q) {
        // xf[m]: step 4G - 4 + m
        float xf[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          xf[2 * m] = bf16_lo(xv[q][m]);
          xf[2 * m + 1] = bf16_hi(xv[q][m]);
        }
        float yv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float acc = f[q][0][r] * xf[4 + r];
#pragma unroll
          for (int k = 1; k < W; ++k) {
            const float xk = (!POS || k <= pos4[r]) ? xf[4 + r - k] : 0.f;
            acc = fmaf(f[q][k][r], xk, acc);
          }
          yv[r] = acc;
        }
        // steps 4G + r of channel 16q + j, two steps per packed dword
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const uint32_t pk = pack_bf16x2(yv[r], yv[r + 1]);
          ys[wave][4 * G + r][16 * q + j].bits = (uint16_t)(pk & 0xffffu);
          ys[wave][4 * G + r + 1][16 * q + j].bits = (uint16_t)(pk >> 16);
        }
      }
      wave_lds_sync();
      const int tbase = tblk0 + 16 * blk;  // step of row 0 of this block
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + lr;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&ys[wave][r][8 * lp]);
        buf_store16<true>(yb, wave_ok ? (uint32_t)(tbase + r) * row_bytes + (uint32_t)((cw0 + 8 * lp) * 2) : kOutOfRange, v);
      }
      wave_lds_sync();  // the y tile and the other x slot are written again by the next block
      // refill slot i with block blk + PF (the x ring entry was staged above)
      load_x(blk + PF, xr[i]);
      load_zp(blk + PF, i);
    });
  }
}

// ----------------------------------------------------------------------------- backward: dx and dU

// LDS row pitch (bf16 elements) of the per-wave transposed staging tiles: 32 steps
// plus padding that spreads consecutive rows over the banks.
constexpr int kStagePitch = 40;

// Staging rows. One ds_write_b16 of a wave writes the same (channel, tap) or rank
// for the four lane groups g; their rows are placed 2 apart (80 dwords of pitch,
// 8 banks apart) so the four 8-dword runs of one write fall on disjoint banks.
// g tile: column q = ch*W + k of lane group g (channel 4g + ch of the wave).
__device__ __forceinline__ constexpr int g_row(int q, int g) { return (q >> 1) * 8 + 2 * g + (q & 1); }
// inverse: row -> column (4g + ch)*W + k of the wave's 16*W columns
template <int W>
__device__ __forceinline__ constexpr int g_row_column(int row) {
  const int q = 2 * (row >> 3) + (row & 1), g = (row >> 1) & 3;
  return (4 * g + q / W) * W + q % W;
}
// z tile: rank 32s + 8g + jj. A chunk of 32 ranks is permuted as the g tile; the
// 16-rank half chunk of an odd tile count keeps groups 0 and 1 two rows apart.
template <int RT>
__device__ __forceinline__ constexpr int z_row(int s, int g, int jj) {
  return 32 * (s + 1) <= 16 * RT ? 32 * s + (jj >> 1) * 8 + 2 * g + (jj & 1) : 32 * s + (jj >> 1) * 4 + 2 * g + (jj & 1);
}
template <int RT>
__device__ __forceinline__ constexpr int z_row_rank(int row) {
  const int s = row >> 5, rem = row & 31;
  return 32 * (s + 1) <= 16 * RT ? 32 * s + 8 * ((rem >> 1) & 3) + 2 * (rem >> 3) + (rem & 1)
                                 : 32 * s + 8 * ((rem >> 1) & 1) + 2 * (rem >> 2) + (rem & 1);
}


// dU staging of the 32 steps of one stage, per wave. With an even tap count each
// lane's (channel, tap) values of g are contiguous columns of a row-major tile
// ([step][column], the column (4g + ch)*W + k as g is formed, and z as loaded,
// [step][rank]), written 16 bytes at a time and read back transposed; with an odd
// one they are written transposed ([column][step]) 16 bits at a time.
constexpr bool dU_row_stage(int W) { return W % 2 == 0; }

template <int W, int RT, int NW, bool FZ, bool ROW = dU_row_stage(W)>
struct alignas(16) DxdUShared {
  // g (hi, lo): rows step, or rows g_row()
  bf16_t g_t[NW][2][ROW ? 32 : 16 * W][ROW ? 16 * W + 8 : kStagePitch];
  // z: rows step, or rows z_row()
  bf16_t z_t[NW][ROW ? 32 : 16 * RT][ROW ? 16 * RT + 8 : kStagePitch];
  // fused dz: per wave, the partial of one block of 16 steps; two buffers by block parity
  float dz[FZ ? 2 : 1][FZ ? NW : 1][FZ ? 16 : 1][FZ ? 16 * RT + 4 : 1];
};

// Block: NW channel tiles of 16 channels (tile w: channels cblk*16*NW + 16w .. +15; lane
// (t, g) holds channels +4g .. +4g+3), walking steps [ta, tb) of one sequence 16 at a
// time, with the x, dy and z rows of the next PF blocks in flight (PF even).
// dx: f*dy at step t is moved back by k steps (DPP) and summed; the last steps of
//     each block of 16 are completed by the next block, and the block after the range
//     completes its last one.
// dU: g (as bf16 hi + lo) is staged transposed in LDS with z, 32 steps at a time, so the
//     contraction over steps runs on the matrix cores with the partial sums for the
//     wave's 16*W columns held in accumulators across the whole range.
// dz (FZ): g is already laid out step-major with the lane's (channel, tap) pairs
//     in-lane, which is the B operand of dz^T = U . g^T; the U operands of the wave's
//     channels stay in registers. The NW waves' partial sums are added through LDS and
//     the block writes one partial per channel block.
// TS = 2 (without FZ): two waves per channel tile, each forming g and dU for half of
//     the taps (the first one also dx), which halves the dU accumulators and staging
//     tiles per wave so that two waves fit on a SIMD when R*W is large.
template <int W, int KS, int RT, int PF, int NW, bool FZ, int TS, bool POS>
__global__ __launch_bounds__(64 * NW * TS) void lowrank_dxdU_kernel(LowrankArgs a) {
  static_assert(PF % 2 == 0, "the prefetch ring covers whole 32-step stages");
  static_assert(TS == 1 || (!FZ && W % TS == 0), "tap halves only without fused dz");
  constexpr int WT = W / TS;          // taps of g and dU per wave
  constexpr int WP = (WT + 1) & ~1;   // (channel, tap) pairs per channel in the dz operands
  constexpr int KB = WP / 2;          // 4 channels * WP = 8*KB values per lane
  constexpr bool kStreamOut = W * KS <= 4;  // non-temporal dx stores, as in the forward
  constexpr bool kRowStage = dU_row_stage(WT);
  __shared__ DxdUShared<WT, RT, NW * TS, FZ> sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = lane & 15, g = lane >> 4;
  const int ct = wave % NW, th = wave / NW;  // channel tile, tap part
  const uint32_t cblk = blockIdx.x % a.n_cblk;
  const uint32_t rest = blockIdx.x / a.n_cblk;
  const int64_t split = rest % a.n_split, b = rest / a.n_split;
  const int64_t T = a.T, D = a.D, DW = D * W;
  const int R = a.R;
  const int64_t ta = split * a.split_len;
  const int64_t tb = ta + a.split_len < T ? ta + a.split_len : T;
  const int64_t cw0 = (int64_t)cblk * 16 * NW + ct * 16;
  const int64_t cl = cw0 + 4 * g;
  const bool lane_ok = cl < D;  // D is a multiple of 4
  // one past the last step whose dy and z are read: the block after the range reaches
  // W-1 steps past tb
  const int itb = (int)tb;
  const int tdy = (int)(tb + 16 < T ? tb + 16 : T);
  // Resources that end at the last row each tensor is accessed at (x, dx: tb; dy, z:
  // tdy): rows past it read zero (stores are dropped) without a compare. Offsets are
  // 32-bit (each per-sequence range is below 2 GiB), lanes past D start at kOutOfRange.
  const buf_t xb = make_buf(static_cast<const bf16_t*>(a.x) + b * T * D, (uint64_t)(tb * D * 2));
  const buf_t dyb = make_buf(static_cast<const bf16_t*>(a.dy) + b * T * D, (uint64_t)tdy * D * 2);
  const buf_t zb = make_buf(static_cast<const bf16_t*>(a.z) + b * T * R, (uint64_t)tdy * R * 2);
  const buf_t ub = make_buf(a.U, (uint64_t)(R * DW * 2));
  const buf_t dxb = make_buf(static_cast<bf16_t*>(a.out) + b * T * D, (uint64_t)(tb * D * 2));
  const buf_t pb = make_buf(POS ? a.pos + b * T : nullptr, POS ? (uint64_t)tdy * 4 : 0);
  const float res = a.residual ? 1.f : 0.f;
  const bool dx_wave = TS == 1 || th == 0;  // wave-uniform
  auto& gT = sh.g_t[wave];
  auto& zT = sh.z_t[wave];
  const uint32_t row_bytes = (uint32_t)(D * 2);
  const uint32_t lane_base = lane_ok ? (uint32_t)(cl * 2) : kOutOfRange;
  auto row_at = [&](int t) -> uint32_t { return (uint32_t)t * row_bytes + lane_base; };  // t >= 0

  bf16x8_t ua[W][KS];  // tile row m = channel cw0 + m
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int s = 0; s < KS; ++s) ua[k][s] = load_ut<W>(ub, DW, cw0 + tl, dx_wave && cw0 + tl < D, k, s, g, R);
  // dz operands: rank 16m + tl, this lane group's (channel, tap) pairs ch*WP + k
  bf16x8_t ud[FZ ? RT : 1][KB];
  if constexpr (FZ) {
#pragma unroll
    for (int m = 0; m < RT; ++m) {
      const int r = 16 * m + tl;
      const int64_t ubase = (int64_t)r * DW + cl * W;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u32x4_t q;
        uint32_t* w = reinterpret_cast<uint32_t*>(&q);
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
          uint32_t v2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int col = 8 * kb + jj + e, ch = col / WP, k = col % WP;
            v2[e] = (k < W) ? buf_load2(ub, (lane_ok && r < R) ? (uint32_t)((ubase + ch * W + k) * 2) : kOutOfRange) : 0u;
          }
          w[jj / 2] = v2[0] | (v2[1] << 16);
        }
        ud[m][kb] = as_bf16x8(q);
      }
    }
  }
  // fused dz: this (channel block, sequence)'s partial [T][R] (fp32)
  const buf_t dzb = make_buf(FZ ? a.dz_part + ((int64_t)cblk * a.B + b) * T * R : nullptr, FZ ? (uint64_t)(T * R * 4) : 0);

  f32x4_t accU[RT][WT];
#pragma unroll
  for (int m = 0; m < RT; ++m)
#pragma unroll
    for (int n = 0; n < WT; ++n) accU[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Ring of PF slots as in the forward: x of block s in slot s % PF, loaded while block
  // s-PF+1 is computed; dy and z of block s loaded while block s-PF is computed.
  const int nsteps = (int)((tb - ta + 15) / 16);  // blocks of 16 steps with outputs
  const int t0 = (int)ta + tl;
  uint32_t xr[PF][2], dyr[PF][2];
  bf16x8_t zr[PF][KS];
  int pr[PF];  // positions, with dy (POS)
  load_row<2>(xb, t0 >= 16 ? row_at(t0 - 16) : kOutOfRange, xr[PF - 1]);
#pragma unroll
  for (int j = 0; j < PF - 1; ++j) load_row<2>(xb, row_at(t0 + 16 * j), xr[j]);
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    load_row<2>(dyb, row_at(t0 + 16 * j), dyr[j]);
    load_z<KS>(zb, t0 + 16 * j, true, R, g, zr[j]);
    pr[j] = POS ? load_pos(pb, t0 + 16 * j) : 0;
  }
  // filters of block s: f[k] = U_k^T z (M = channel, N = step); computed one block
  // ahead (where the registers allow) so the matrix-core latency overlaps the
  // previous block's vector work
  constexpr bool kAhead = TS == 1 && RT * W <= 32;
  auto filters = [&](const bf16x8_t (&zs)[KS], f32x4_t (&f)[W]) {
#pragma unroll
    for (int k = 0; k < W; ++k) {
      // the residual rides on tap 0's accumulator: dx gets (f_0 + residual) * dy
      f[k] = k == 0 ? f32x4_t{res, res, res, res} : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) f[k] = mfma_16x16x32(ua[k][s], zs[s], f[k]);
    }
  };
  f32x4_t fc[W];
  if constexpr (kAhead) filters(zr[0], fc);
  // Drain the prologue loads once: the compiler's wait counts at the loop head must
  // hold on entry too, and a prologue issued in another order than the ring refills
  // otherwise forces near-full drains at every pass of the loop.
  __builtin_amdgcn_s_waitcnt(0);
  float dxc[4] = {0.f, 0.f, 0.f, 0.f};  // pending dx of the previous 16 steps
  // Whole rings without branches: blocks past nsteps read zeros (g and dz are masked
  // past tb) and store nothing; a pass always ends on a complete 32-step stage.
  int s0 = 0;
  for (; s0 < nsteps; s0 += PF) {
    static_for<0, PF>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int jp = (j + PF - 1) % PF;
      constexpr int half = j & 1;  // s0 is a multiple of PF, PF even
      const int step = s0 + j;
      const int t = t0 + 16 * step;
      float dyf[4];
      unpack_row<2>(dyr[j], dyf);
      if (dx_wave) {
        if constexpr (!kAhead) filters(zr[j], fc);
        // dx: p_k = f_k * dy at step t contributes to dx at step t-k
        float cur[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = fc[0][i] * dyf[i];
        static_for<1, W>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          const bool on = !POS || k <= pr[j];  // tap k of step t exists
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = on ? fc[k][i] * dyf[i] : 0.f;
            cur[i] += lanes_up<k>(p);         // to step t-k in this block
            dxc[i] += lanes_down<16 - k>(p);  // to step t-k in the previous block
          }
        });
        store_row<2, kStreamOut>(dxb, step > 0 ? row_at(t - 16) : kOutOfRange, dxc);  // block -1 is outside [ta, tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dxc[i] = cur[i];
        if constexpr (kAhead) filters(zr[(j + 1) % PF], fc);  // next block's filters (its z is resident)
      }
      // g, its staging for dU and dz, for taps K0 .. K0+WT-1
      auto g_part = [&](auto k0c) {
        constexpr int K0 = decltype(k0c)::value;
        // g[ch*WP + kk] = dy * x[t-K0-kk] for steps inside [ta, tb) (padding tap zero)
        const float rin = t < itb ? 1.f : 0.f;
        float gv[4 * WP];
        static_for<0, WT>([&](auto kc) {
          constexpr int kk = decltype(kc)::value;
          constexpr int k = K0 + kk;
          uint32_t xk[2];
          if constexpr (k == 0) {
            xk[0] = xr[j][0];
            xk[1] = xr[j][1];
          } else {
            xk[0] = rows_back<k>(xr[jp][0], xr[j][0]);
            xk[1] = rows_back<k>(xr[jp][1], xr[j][1]);
          }
          float xkf[4];
          unpack_row<2>(xk, xkf);
          const bool on = !POS || k == 0 || k <= pr[j];
#pragma unroll
          for (int i = 0; i < 4; ++i) gv[i * WP + kk] = on ? rin * dyf[i] * xkf[i] : 0.f;
        });
        if constexpr (WP != WT) {
#pragma unroll
          for (int i = 0; i < 4; ++i) gv[i * WP + WT] = 0.f;
        }
        u32x4_t ghi[KB], glo[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          bf16x8_t h8, l8;
          split_hi_lo(gv + 8 * kb, h8, l8);
          ghi[kb] = __builtin_bit_cast(u32x4_t, h8);
          glo[kb] = __builtin_bit_cast(u32x4_t, l8);
        }
        // dz^T[r, t] over this wave's 16 channels (g is the B operand as it stands)
        f32x4_t dzacc[FZ ? RT : 1];
        if constexpr (FZ) {
#pragma unroll
          for (int m = 0; m < RT; ++m) {
            dzacc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              dzacc[m] = mfma_16x16x32(ud[m][kb], as_bf16x8(ghi[kb]), dzacc[m]);
              dzacc[m] = mfma_16x16x32(ud[m][kb], as_bf16x8(glo[kb]), dzacc[m]);
            }
          }
        }
        // stage g and z for dU: step slot 16*half + tl
        const int col_t = 16 * half + tl;
        if constexpr (kRowStage) {
          // the lane's 4*WT values of g are columns 4g*WT .. of its step's row
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            *reinterpret_cast<u32x4_t*>(&gT[0][col_t][4 * g * WT + 8 * kb]) = ghi[kb];
            *reinterpret_cast<u32x4_t*>(&gT[1][col_t][4 * g * WT + 8 * kb]) = glo[kb];
          }
#pragma unroll
          for (int s = 0; s < KS; ++s)  // (past tb g is zero, so z needs no mask)
            if (32 * s + 8 * g < 16 * RT)
              *reinterpret_cast<u32x4_t*>(&zT[col_t][32 * s + 8 * g]) = __builtin_bit_cast(u32x4_t, zr[j][s]);
        } else {
#pragma unroll
          for (int ch = 0; ch < 4; ++ch)
#pragma unroll
            for (int kk = 0; kk < WT; ++kk) {
              const int v = ch * WP + kk, row = g_row(ch * WT + kk, g);
              const uint32_t hw = reinterpret_cast<const uint32_t*>(&ghi[v / 8])[(v % 8) / 2];
              const uint32_t lw = reinterpret_cast<const uint32_t*>(&glo[v / 8])[(v % 8) / 2];
              gT[0][row][col_t].bits = (uint16_t)((v & 1) ? hw >> 16 : hw & 0xffffu);
              gT[1][row][col_t].bits = (uint16_t)((v & 1) ? lw >> 16 : lw & 0xffffu);
            }
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const u32x4_t q = __builtin_bit_cast(u32x4_t, zr[j][s]);
            const uint32_t zw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              if (32 * s + 8 * g + jj < 16 * RT)
                zT[z_row<RT>(s, g, jj)][col_t].bits = (uint16_t)((jj & 1) ? zw[jj / 2] >> 16 : zw[jj / 2] & 0xffffu);
            }
          }
        }
        if constexpr (half == 1) {
          wave_lds_sync();
          // dU[r, col] += sum over these 32 steps of z[step, r] * g[step, col]; with the
          // row tiles lane (G, j) = (g, tl) takes steps 8G .. 8G+7 of column j (or rank j)
          // of each 16-column tile as its K slots, through two transposing reads
          const int r4 = tl >> 2, q4 = tl & 3;
#pragma unroll
          for (int m = 0; m < RT; ++m) {
            const bf16x8_t za = kRowStage
                                    ? lds_read_tr8(&zT[8 * g + r4][16 * m + 4 * q4], 16 * RT + 8)
                                    : as_bf16x8(*reinterpret_cast<const u32x4_t*>(&zT[16 * m + tl][8 * g]));
#pragma unroll
            for (int n = 0; n < WT; ++n) {
              bf16x8_t gh, gl;
              if constexpr (kRowStage) {
                gh = lds_read_tr8(&gT[0][8 * g + r4][16 * n + 4 * q4], 16 * WT + 8);
                gl = lds_read_tr8(&gT[1][8 * g + r4][16 * n + 4 * q4], 16 * WT + 8);
              } else {
                gh = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&gT[0][16 * n + tl][8 * g]));
                gl = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&gT[1][16 * n + tl][8 * g]));
              }
              accU[m][n] = mfma_16x16x32(za, gh, accU[m][n]);
              accU[m][n] = mfma_16x16x32(za, gl, accU[m][n]);
            }
          }
          wave_lds_sync();
        }
        if constexpr (FZ) {
          // the sum of dz over the block's waves
#pragma unroll
          for (int m = 0; m < RT; ++m) *reinterpret_cast<f32x4_t*>(&sh.dz[half][wave][tl][16 * m + 4 * g]) = dzacc[m];
          // One barrier per block of 16 steps: the buffer of this parity is written
          // again two blocks later, after the next block's barrier.
          __syncthreads();
          const int tstep0 = (int)ta + 16 * step;
          constexpr int NE = 16 * 16 * RT;  // (step, padded rank) elements
#pragma unroll
          for (int e0 = 0; e0 < NE; e0 += 64 * NW) {
            const int e = e0 + (int)threadIdx.x;
            const int tr = (e / (16 * RT)) & 15, r = e % (16 * RT);
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += sh.dz[half][w][tr][r];
            const bool ok = (e0 + 64 * NW <= NE || e < NE) && r < R && tstep0 + tr < itb;
            buf_store_f32(dzb, ok ? (uint32_t)((tstep0 + tr) * R + r) * 4u : kOutOfRange, sum);
          }
        }
      };
      if constexpr (TS == 1) {
        g_part(std::integral_constant<int, 0>{});
      } else {
        if (th == 0)
          g_part(std::integral_constant<int, 0>{});
        else
          g_part(std::integral_constant<int, WT>{});
      }
      // refill: x of block step+PF-1 into the previous block's slot; dy, z of block step+PF into this one
      load_row<2>(xb, row_at(t + 16 * (PF - 1)), xr[jp]);
      load_row<2>(dyb, row_at(t + 16 * PF), dyr[j]);
      load_z<KS>(zb, t + 16 * PF, true, R, g, zr[j]);
      if constexpr (POS) pr[j] = load_pos(pb, t + 16 * PF);
    });
  }
  // block s0 (slot 0) only completes the dx of block s0-1 with its first steps
  if (dx_wave) {
    if constexpr (!kAhead) filters(zr[0], fc);
    float dyf[4];
    unpack_row<2>(dyr[0], dyf);
    static_for<1, W>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const bool on = !POS || k <= pr[0];
#pragma unroll
      for (int i = 0; i < 4; ++i) dxc[i] += lanes_down<16 - k>(on ? fc[k][i] * dyf[i] : 0.f);
    });
    store_row<2, kStreamOut>(dxb, s0 > 0 ? row_at(t0 + 16 * (s0 - 1)) : kOutOfRange, dxc);
  }
  // partial dU of this (sequence, split): accumulator row 16m + 4g + i is rank
  // 16m + 4g + i (row tiles) or z_row_rank(.), column 16n + tl is the wave's column
  // 16n + tl (row tiles) or g_row_column(.), = (4g' + ch)*WT + kk: channel
  // cw0 + 4g' + ch, tap th*WT + kk
  float* dst = a.dU_part + (b * a.n_split + split) * (int64_t)R * DW + cw0 * W;
#pragma unroll
  for (int n = 0; n < WT; ++n) {
    const int lc = kRowStage ? 16 * n + tl : g_row_column<WT>(16 * n + tl);
    const int ch16 = lc / WT, col = ch16 * W + th * WT + lc % WT;
    const bool col_ok = cw0 + ch16 < D;
#pragma unroll
    for (int m = 0; m < RT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = kRowStage ? 16 * m + 4 * g + i : z_row_rank<RT>(16 * m + 4 * g + i);
        if (r < R && col_ok) dst[(int64_t)r * DW + col] = accU[m][n][i];
      }
  }
}

// ----------------------------------------------------------------------------- backward: dz

// Block: 4 waves, each over MB*16 consecutive steps of one sequence (the block covers
// 64*MB steps), looping over one channel split 16 channels at a time. For every
// 16-channel chunk the U operands (16 ranks x 8 (channel, tap) columns per lane) are
// applied to all MB step blocks; dz accumulates across the chunks.
// The four waves walk the same chunks, so the U operands of a chunk are fetched once
// per block: each wave loads a quarter of the next chunk's operands from global memory
// while the current chunk is computed and writes them to an LDS double buffer (one
// barrier per chunk). The x and dy rows of the next chunk are prefetched as well.
// Columns within a lane are (channel, tap) pairs ordered ch*WP + k, WP = W rounded up
// to even (the padding tap is zero), so each MFMA takes 8 of the lane's own values.
template <int W, int RT, int MB, bool POS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void lowrank_dz_kernel(LowrankArgs a) {
  constexpr int WP = (W + 1) & ~1;
  constexpr int KB = WP / 2;  // 4 channels * WP columns = 8*KB per lane
  constexpr int NOP = RT * KB;          // U operands per lane and chunk
  constexpr int NOW = (NOP + 3) / 4;    // of which each wave fetches at most NOW
  __shared__ u32x4_t ush[2][NOP][64];
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
  const buf_t xb = make_buf(static_cast<const bf16_t*>(a.x) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t dyb = make_buf(static_cast<const bf16_t*>(a.dy) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t ub = make_buf(a.U, (uint64_t)(R * DW * 2));

  f32x4_t acc[MB][RT];
#pragma unroll
  for (int h = 0; h < MB; ++h)
#pragma unroll
    for (int m = 0; m < RT; ++m) acc[h][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // positions of the wave's steps (POS): the same for every channel chunk
  int pz[MB];
  {
    const buf_t pb = make_buf(POS ? a.pos + b * T : nullptr, POS ? (uint64_t)(T * 4) : 0);
#pragma unroll
    for (int h = 0; h < MB; ++h) pz[h] = POS ? load_pos(pb, (int)(tw0 + 16 * h + tl)) : 0;
  }

  // x rows tw0-16 .. tw0+16*MB-1 (block 0 is the halo) and dy rows of one chunk; per-sequence
  // ranges are below 2 GiB, so offsets are 32-bit and out-of-range rows read zeros.
  const uint32_t row_bytes = (uint32_t)(D * 2);
  const int iT = (int)T, itw = (int)tw0 + tl;
  auto load_chunk = [&](int64_t c0, uint32_t (&xv)[MB + 1][2], uint32_t (&dyv)[MB][2]) {
    const uint32_t cl = (uint32_t)(c0 + 4 * g);
    const bool ok = (int64_t)cl < c_end;
#pragma unroll
    for (int h = 0; h <= MB; ++h) {
      const int t = itw + 16 * (h - 1);
      const uint32_t off = (ok & (t >= 0) & (t < iT)) ? (uint32_t)t * row_bytes + cl * 2u : kOutOfRange;
      load_row<2>(xb, off, xv[h]);
      if (h > 0) load_row<2>(dyb, off, dyv[h - 1]);
    }
  };
  // U operand o = m*KB + kb of chunk c0 for this lane: rank 16m + tl, columns 8kb.. of
  // this lane group's (channel, tap) pairs
  auto load_operand = [&](int64_t c0, int o) -> u32x4_t {
    const int m = o / KB, kb = o % KB;
    const int64_t cl = c0 + 4 * g;
    const bool ok = cl < c_end && 16 * m + tl < R;
    const int64_t ubase = (int64_t)(16 * m + tl) * DW + cl * W;
    if constexpr (WP == W) {
      return buf_load16(ub, ok ? (uint32_t)((ubase + 8 * kb) * 2) : kOutOfRange);
    } else {
      u32x4_t q;
      uint32_t* w = reinterpret_cast<uint32_t*>(&q);
#pragma unroll
      for (int jj = 0; jj < 8; jj += 2) {
        uint32_t v2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int col = 8 * kb + jj + e, ch = col / WP, k = col % WP;
          v2[e] = (k < W) ? buf_load2(ub, ok ? (uint32_t)((ubase + ch * W + k) * 2) : kOutOfRange) : 0u;
        }
        w[jj / 2] = v2[0] | (v2[1] << 16);
      }
      return q;
    }
  };
  auto fetch_operands = [&](int64_t c0, u32x4_t (&pre)[NOW]) {
#pragma unroll
    for (int i = 0; i < NOW; ++i) {
      const int o = wave + 4 * i;
      pre[i] = o < NOP ? load_operand(c0, o < NOP ? o : 0) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_operands = [&](int buf, const u32x4_t (&pre)[NOW]) {
#pragma unroll
    for (int i = 0; i < NOW; ++i) {
      const int o = wave + 4 * i;
      if (o < NOP) ush[buf][o][lane] = pre[i];
    }
  };

  // Every wave walks every chunk (rows past T read zeros) so that the barriers match.
  {
    u32x4_t pre[NOW];
    fetch_operands(c_begin, pre);
    store_operands(0, pre);
  }
  __syncthreads();
  uint32_t xv[2][MB + 1][2], dyv[2][MB][2];
  load_chunk(c_begin, xv[0], dyv[0]);
  for (int64_t c00 = c_begin; c00 < c_end; c00 += 32) {
    static_for<0, 2>([&](auto pc) {
      constexpr int P = decltype(pc)::value;
      const int64_t c0 = c00 + 16 * P;
      if (c0 < c_end) {
        load_chunk(c0 + 16, xv[1 - P], dyv[1 - P]);  // next chunk (past the split: zeros)
        u32x4_t pre[NOW];
        fetch_operands(c0 + 16, pre);
#pragma unroll
        for (int h = 0; h < MB; ++h) {
          float dyf[4], gv[4 * WP];
          unpack_row<2>(dyv[P][h], dyf);
          {
            float xf[4];
            unpack_row<2>(xv[P][h + 1], xf);
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[i * WP] = dyf[i] * xf[i];
          }
          static_for<1, W>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            uint32_t xk[2] = {rows_back<k>(xv[P][h][0], xv[P][h + 1][0]), rows_back<k>(xv[P][h][1], xv[P][h + 1][1])};
            float xkf[4];
            unpack_row<2>(xk, xkf);
            const bool on = !POS || k <= pz[h];
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[i * WP + k] = on ? dyf[i] * xkf[i] : 0.f;
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
              // operands re-read from LDS per step block: registers stay free for the x, dy prefetch
              const bf16x8_t u = as_bf16x8(ush[P][m * KB + kb][lane]);
              acc[h][m] = mfma_16x16x32(u, ghi, acc[h][m]);
              acc[h][m] = mfma_16x16x32(u, glo, acc[h][m]);
            }
          }
        }
        // the other buffer was last read in the previous chunk, before its barrier
        store_operands(1 - P, pre);
        __syncthreads();
      }
    });
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
