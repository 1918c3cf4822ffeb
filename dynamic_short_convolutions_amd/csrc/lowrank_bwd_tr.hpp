// Low-rank backward, dx and dU, for ranks whose dz runs in its own pass
// (R > 32): the x, dy and z rows a workgroup needs are staged in LDS once, and
// the work is split by role between the two waves that share a 16-channel tile.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", technical
// summary page, section Metodologia, low-rank factorisation, and the
// fused-kernel section; the gradients are the chain rule on the forward):
//   f[t,c,k]  = sum_r z[t,r] U[r, c*W+k]                   (regenerated, never stored)
//   dx[s,c]   = residual*dy[s,c] + sum_k f[s+k,c,k] dy[s+k,c]
//   dU[r,c*W+k] = sum_t z[t,r] g[t,c,k],  g[t,c,k] = dy[t,c] x[t-k,c]
//
// Workgroup: 8 waves over 64 channels (4 tiles of 16) and one time split of one
// sequence, walked in blocks of 32 steps. Each block's x rows (t0-8 .. t0+31),
// dy and z rows (t0 .. t0+39) are loaded cooperatively (16 bytes per lane), two
// blocks ahead, into one of two LDS stages while the other stage is computed on;
// one barrier per block.
//
// Both roles work "time in lane": lane (j, G) = (lane % 16, lane / 16) owns
// channel 16w + j of its wave's tile. Transposing LDS reads
// (ds_read_b64_tr_b16: lane 4r+q of a 16-lane group names row r, columns
// 4q..4q+3 of a row-major tile; lane j receives column j of those 4 rows) hand
// it consecutive steps of its channel, so no value moves between lanes.
// Waves 0-3 (g and dU): the lane's steps are t0 + 8G .. t0 + 8G + 7; g for one
// tap is formed from registers, and its 8 steps are the K slots of the dU
// contraction's B operand as they stand; z^T, the A operand, comes from the same
// reads of the z tile. g = dy*x (16 significant bits) enters as bf16 hi + lo.
// Waves 4-7 (filters and dx): the filter contraction runs with M = step, N =
// channel, K = rank, and for tap k its A operand is the z rows k steps later, so
// lane (j, G) receives f[s+k, c, k] for its steps s = 16h + 4G .. +3 of each half
// h of the block. With dy[s+k] from transposing reads, dx[s] is W products added
// in tap order, all in the lane; a block's dx is complete within the block (its z
// and dy rows reach 8 steps past it). The four waves put their dx into a shared
// 32 x 64 tile that they store, whole 128-byte lines, in the next block.
//
// Dense sequences only (packed ones take the two-wave kernel in lowrank_mfma.hpp).
#pragma once

#include "lowrank_mfma.hpp"

namespace dsc {

namespace bwd_tr {
constexpr int kTiles = 4;            // 16-channel tiles per workgroup
constexpr int kBlk = 32;             // steps per block
constexpr int kXRows = kBlk + 8;     // x rows t0-8 .. t0+31 (tap 7 of step t0 reaches t0-7)
constexpr int kYRows = kBlk + 8;     // dy and z rows t0 .. t0+39 (dx of step t0+31 reaches t0+38)
constexpr int kPitch = 16 * kTiles + 8;  // bf16 per staged x / dy row: 64 channels + 16 bytes
constexpr int kThreads = 64 * 2 * kTiles;
}  // namespace bwd_tr

template <int KS>
struct alignas(16) BwdTrStage {
  bf16_t x[bwd_tr::kXRows][bwd_tr::kPitch];
  bf16_t dy[bwd_tr::kYRows][bwd_tr::kPitch];
  // ranks padded to the filter contraction's K (zeros past R), rows of 32*KS + 16 values:
  // the dx waves read 16 consecutive rows at one column per instruction (16 bytes a
  // lane), and measured per kernel, LDS bank-conflict cycles at the long-sequence
  // workload were 9.0e7 with 8 values of padding, 2.4e8 with none, 2.3e7 with 16
  bf16_t z[bwd_tr::kYRows][32 * KS + 16];
};

template <int W, int KS, int RT>
__global__ __launch_bounds__(bwd_tr::kThreads) void lowrank_dxdU_tr_kernel(LowrankArgs a) {
  using namespace bwd_tr;
  constexpr int ZC = 4 * KS;  // 16-byte chunks per staged z row
  __shared__ BwdTrStage<KS> st[2];
  // dx of a block (32 steps x 64 channels), by block parity
  __shared__ __attribute__((aligned(16))) bf16_t dxs[2][kBlk][kPitch];

  const int lane = threadIdx.x & 63;
  const uint32_t cblk = blockIdx.x % a.n_cblk;
  const uint32_t rest = blockIdx.x / a.n_cblk;
  const int64_t split = rest % a.n_split, b = rest / a.n_split;
  const int64_t T = a.T, D = a.D, DW = D * W;
  const int R = a.R;
  const int64_t ta = split * a.split_len;
  const int64_t tb = ta + a.split_len < T ? ta + a.split_len : T;
  const int nblk = (int)((tb - ta + kBlk - 1) / kBlk);
  const int64_t c0 = (int64_t)cblk * 16 * kTiles;
  const int itb = (int)tb;
  // rows past these read zero: x to the end of the sequence; dy and z to one block past
  // the split (the completion of the last dx rows)
  const int tdy = (int)(tb + kBlk < T ? tb + kBlk : T);
  const buf_t xb = make_buf(static_cast<const bf16_t*>(a.x) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t dyb = make_buf(static_cast<const bf16_t*>(a.dy) + b * T * D, (uint64_t)tdy * D * 2);
  const buf_t zb = make_buf(static_cast<const bf16_t*>(a.z) + b * T * R, (uint64_t)tdy * R * 2);

  // Cooperative staging in units of 64 chunks (one per lane; a chunk is 8 channels or
  // ranks of one row): units 0-4 are the 40 x rows, 5-9 the 40 dy rows, then the z rows
  // (the last z unit may be partly idle). Unit u is loaded by wave u % 8 in slot u / 8,
  // so the tensor, and with it the buffer resource, is uniform over each wave.
  constexpr int kXU = kXRows * 8 / 64, kYU = kYRows * 8 / 64, kZU = (kYRows * ZC + 63) / 64;
  constexpr int NPF = (kXU + kYU + kZU + 7) / 8;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint32_t q_lds[NPF], q_base[NPF], q_row_bytes[NPF];
  int q_trow[NPF];  // the row's step relative to t0
  buf_t q_buf[NPF];
  bool q_on[NPF];
#pragma unroll
  for (int i = 0; i < NPF; ++i) {
    const int u = 8 * i + wv;  // wave-uniform
    const int q = 64 * u + lane;
    q_on[i] = u < kXU + kYU + kZU;
    q_lds[i] = 0;
    q_base[i] = kOutOfRange;
    q_row_bytes[i] = 0;
    q_trow[i] = 0;
    q_buf[i] = xb;
    if (u < kXU) {
      const int row = q / 8, ch = 8 * (q % 8);
      q_lds[i] = (uint32_t)(reinterpret_cast<uintptr_t>(&st[0].x[row][ch]) - reinterpret_cast<uintptr_t>(&st[0]));
      q_trow[i] = row - 8;
      q_row_bytes[i] = (uint32_t)(D * 2);
      q_base[i] = c0 + ch < D ? (uint32_t)((c0 + ch) * 2) : kOutOfRange;
    } else if (u < kXU + kYU) {
      const int qq = q - kXU * 64, row = qq / 8, ch = 8 * (qq % 8);
      q_lds[i] = (uint32_t)(reinterpret_cast<uintptr_t>(&st[0].dy[row][ch]) - reinterpret_cast<uintptr_t>(&st[0]));
      q_trow[i] = row;
      q_row_bytes[i] = (uint32_t)(D * 2);
      q_base[i] = c0 + ch < D ? (uint32_t)((c0 + ch) * 2) : kOutOfRange;
      q_buf[i] = dyb;
    } else if (q_on[i]) {
      const int qq = q - (kXU + kYU) * 64, row = qq / ZC, rk = 8 * (qq % ZC);
      q_on[i] = row < kYRows;  // lanes past the last z row stay idle
      const int rw = q_on[i] ? row : 0;
      q_lds[i] = (uint32_t)(reinterpret_cast<uintptr_t>(&st[0].z[rw][rk]) - reinterpret_cast<uintptr_t>(&st[0]));
      q_trow[i] = rw;
      q_row_bytes[i] = (uint32_t)(R * 2);
      q_base[i] = (q_on[i] && rk < R) ? (uint32_t)(rk * 2) : kOutOfRange;  // ranks past R stage zeros
      q_buf[i] = zb;
    }
  }
  const uint32_t stage_bytes = (uint32_t)sizeof(BwdTrStage<KS>);
  // Block n's rows are loaded two blocks ahead, at the start of iteration n-2, into
  // register set n % 2, and written to stage n % 2 at the end of iteration n-1 (that
  // stage held block n-2, whose readers passed the barrier ending iteration n-2).
  // Two blocks of loads are thus in flight while a block is computed: with one, each
  // block waited on a full memory round trip.
  u32x4_t pre[2][NPF];
  auto issue = [&](int blk, u32x4_t (&P)[NPF]) {
    const int t0 = (int)ta + kBlk * blk;
    // every slot issues its load (an idle one reads out of range: zeros, no traffic), so
    // the number of loads in flight is known at compile time and the wait before a
    // commit leaves the newer block's loads outstanding
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int t = t0 + q_trow[i];
      const uint32_t off = (t >= 0 && q_base[i] != kOutOfRange) ? (uint32_t)t * q_row_bytes[i] + q_base[i] : kOutOfRange;
      P[i] = buf_load16(q_buf[i], off);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads at the top of the block
  };
  auto commit = [&](int s, const u32x4_t (&P)[NPF]) {
#pragma unroll
    for (int i = 0; i < NPF; ++i)
      if (q_on[i]) *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(&st[0]) + s * stage_bytes + q_lds[i]) = P[i];
  };
  // iteration blk: loads of block blk+2 into set blk % 2, compute on stage blk % 2,
  // block blk+1 from set (blk+1) % 2 into stage (blk+1) % 2, barrier. The loop body
  // is unrolled by two so that every register set is named at compile time.
  auto walk = [&](auto&& compute) {
    int blk = 0;
    for (; blk + 1 < nblk; blk += 2) {
      issue(blk + 2, pre[0]);
      compute(blk, st[0]);
      commit(1, pre[1]);
      __syncthreads();
      issue(blk + 3, pre[1]);
      compute(blk + 1, st[1]);
      commit(0, pre[0]);
      __syncthreads();
    }
    if (blk < nblk) {  // an odd block count: the last block, then block nblk into stage 1
      compute(blk, st[0]);
      commit(1, pre[1]);
      __syncthreads();
    }
  };

  issue(0, pre[0]);
  issue(1, pre[1]);
  commit(0, pre[0]);
  __syncthreads();

  if (wv < kTiles) {  // a scalar branch: the role is the wave's
    // ------------------------------------------------------------------ g and dU
    const int w = wv, j = lane & 15, G = lane >> 4;
    const int r4 = (lane & 15) >> 2, q4 = lane & 3;  // this lane's address in a transposing read
    f32x4_t acc[RT][W];
#pragma unroll
    for (int m = 0; m < RT; ++m)
#pragma unroll
      for (int k = 0; k < W; ++k) acc[m][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    walk([&](int blk, const BwdTrStage<KS>& S) {
      // x rows 8G .. 8G+15 of the stage (steps t0+8G-8 ..), dy rows 8G .. 8G+7, z^T
      float xv[16], dyv[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint2 v = lds_read_tr(&S.x[8 * G + 4 * u + r4][16 * w + 4 * q4]);
        xv[4 * u + 0] = bf16_lo(v.x); xv[4 * u + 1] = bf16_hi(v.x);
        xv[4 * u + 2] = bf16_lo(v.y); xv[4 * u + 3] = bf16_hi(v.y);
      }
      const int tstep = (int)ta + kBlk * blk + 8 * G;  // step of dyv[0]
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint2 v = lds_read_tr(&S.dy[8 * G + 4 * u + r4][16 * w + 4 * q4]);
        // steps past the split take no part in dU
        dyv[4 * u + 0] = tstep + 4 * u + 0 < itb ? bf16_lo(v.x) : 0.f;
        dyv[4 * u + 1] = tstep + 4 * u + 1 < itb ? bf16_hi(v.x) : 0.f;
        dyv[4 * u + 2] = tstep + 4 * u + 2 < itb ? bf16_lo(v.y) : 0.f;
        dyv[4 * u + 3] = tstep + 4 * u + 3 < itb ? bf16_hi(v.y) : 0.f;
      }
      bf16x8_t za[RT];
#pragma unroll
      for (int m = 0; m < RT; ++m) {
        const uint2 v0 = lds_read_tr(&S.z[8 * G + r4][16 * m + 4 * q4]);
        const uint2 v1 = lds_read_tr(&S.z[8 * G + 4 + r4][16 * m + 4 * q4]);
        za[m] = as_bf16x8(u32x4_t{v0.x, v0.y, v1.x, v1.y});
      }
#pragma unroll
      for (int k = 0; k < W; ++k) {
        float gv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[i] = dyv[i] * xv[i - k + 8];
        bf16x8_t hi, lo;
        split_hi_lo(gv, hi, lo);
        // consecutive MFMAs on different accumulators
#pragma unroll
        for (int m = 0; m < RT; ++m) acc[m][k] = mfma_16x16x32(za[m], hi, acc[m][k]);
#pragma unroll
        for (int m = 0; m < RT; ++m) acc[m][k] = mfma_16x16x32(za[m], lo, acc[m][k]);
      }
    });
    // partial dU of this (sequence, split): lane (j, G) holds rank 16m + 4G + i of
    // channel c0 + 16w + j, tap k
    const int64_t c = c0 + 16 * w + j;
    if (c < D) {
      float* dst = a.dU_part + (b * a.n_split + split) * (int64_t)R * DW + c * W;
#pragma unroll
      for (int m = 0; m < RT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * m + 4 * G + i;
          if (r < R) {
#pragma unroll
            for (int k = 0; k < W; ++k) dst[(int64_t)r * DW + k] = acc[m][k][i];
          }
        }
    }
  } else {
    // ------------------------------------------------------------------ filters and dx
    const int w = wv - kTiles, j = lane & 15, G = lane >> 4;
    const int r4 = j >> 2, q4 = j & 3;  // this lane's address in a transposing read
    const int64_t c = c0 + 16 * w + j;  // this lane's channel
    constexpr bool kStreamOut = W * KS <= 4;
    const buf_t dxb = make_buf(static_cast<bf16_t*>(a.out) + b * T * D, (uint64_t)(tb * D * 2));
    const uint32_t row_bytes = (uint32_t)(D * 2);
    const buf_t ub = make_buf(a.U, (uint64_t)(R * DW * 2));
    const float res = a.residual ? 1.f : 0.f;
    // B operands: U[32s + 8G + jj, c*W + k]
    bf16x8_t ub_op[W][KS];
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
      for (int s = 0; s < KS; ++s) ub_op[k][s] = load_ut<W>(ub, DW, c, c < D, k, s, G, R);
    // 4-row transposing reads covering steps 4G .. 4G + 3 + (W-1) of a half block
    constexpr int NU = (W + 6) / 4;
    // the piece of a dx tile this lane stores: row 8w + lane/8, channels 8*(lane%8) ..
    const int srow = 8 * w + (lane >> 3), spc = lane & 7;
    const uint32_t sbase = c0 + 8 * spc < D ? (uint32_t)((c0 + 8 * spc) * 2) : kOutOfRange;
    auto store_tile = [&](int blk) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&dxs[blk & 1][srow][8 * spc]);
      const int t = (int)ta + kBlk * blk + srow;  // rows past the split are dropped
      buf_store16<kStreamOut>(dxb, sbase != kOutOfRange ? (uint32_t)t * row_bytes + sbase : kOutOfRange, v);
    };
    walk([&](int blk, const BwdTrStage<KS>& S) {
      // the previous block's tile was completed by all four waves before the barrier
      if (blk > 0) store_tile(blk - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // f[k][i] = f[s+k, c, k] for s = 16h + 4G + i; the residual rides on tap 0
        f32x4_t f[W];
#pragma unroll
        for (int k = 0; k < W; ++k) f[k] = k == 0 ? f32x4_t{res, res, res, res} : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int k = 0; k < W; ++k) {
            const bf16x8_t za = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&S.z[16 * h + j + k][32 * s + 8 * G]));
            f[k] = mfma_16x16x32(za, ub_op[k][s], f[k]);
          }
        // dyv[m]: dy at step 16h + 4G + m of channel c
        float dyv[4 * NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const uint2 v = lds_read_tr(&S.dy[16 * h + 4 * G + 4 * u + r4][16 * w + 4 * q4]);
          dyv[4 * u + 0] = bf16_lo(v.x); dyv[4 * u + 1] = bf16_hi(v.x);
          dyv[4 * u + 2] = bf16_lo(v.y); dyv[4 * u + 3] = bf16_hi(v.y);
        }
        float out[4];
        {
          // each product rounded, then added in tap order, as the kernels that move the
          // products between lanes do (packed sequences there give these bits exactly)
#pragma clang fp contract(off)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float acc = f[0][i] * dyv[i];
#pragma unroll
            for (int k = 1; k < W; ++k) acc = acc + f[k][i] * dyv[i + k];
            out[i] = acc;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const uint32_t pk = pack_bf16x2(out[i], out[i + 1]);
          dxs[blk & 1][16 * h + 4 * G + i][16 * w + j].bits = (uint16_t)(pk & 0xffffu);
          dxs[blk & 1][16 * h + 4 * G + i + 1][16 * w + j].bits = (uint16_t)(pk >> 16);
        }
      }
    });
    // the last block's tile (the walk ends with a barrier)
    if (nblk > 0) store_tile(nblk - 1);
  }
}

}  // namespace dsc

namespace dsc {

// ----------------------------------------------------------------------------- dz
// dz[t,r] = sum_{c,k} g[t,c,k] U[r, c*W+k] for ranks whose dz has its own pass.
//
// Block: 8 waves over 256 steps of one sequence (wave w: steps t0 + 32w + 16h + l%16,
// h < 2), walking one channel split. The x and dy rows are staged in LDS 64 channels (one
// 128-byte line of each row) at a time, x as fp32, dy as bf16: a line is consumed
// in one stage (the rows a block reads lie D*2 bytes apart, and lines read a quarter
// at a time were evicted before their next quarter, so each was fetched about four
// times). The stage is computed 16 channels at a time; for each such sub-chunk the U
// operands (16 ranks x 8 (channel, tap) columns per lane, RT*KB of them) are staged
// in their register layout, double-buffered, one barrier per sub-chunk; each operand
// serves a wave's two blocks of 16 steps. The next stage's rows travel in registers
// meanwhile and are written to LDS after its last sub-chunk. A lane reads x[t-k] of its 4 channels straight from LDS for each tap,
// so g costs one multiply and its bf16 hi/lo split per value: no shifts between
// lanes and no per-tap unpacking. The lane's (channel, tap) values are ordered
// ch*WP + k (WP = W rounded up to even, the padding tap zero), 8 per MFMA.
// Dense sequences only (packed ones take lowrank_dz_kernel).
namespace dz_lds {
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMB = 2;                    // blocks of 16 steps per wave
constexpr int kRows = 16 * kMB * kWaves;  // steps per block
constexpr int kCh = 64;             // channels per stage
constexpr int kXPitch = kCh + 4;    // floats
constexpr int kYPitch = kCh + 8;    // bf16
}  // namespace dz_lds

template <int W, int RT>
struct alignas(16) DzLdsShared {
  static constexpr int WP = (W + 1) & ~1;
  static constexpr int KB = WP / 2;
  float x[dz_lds::kRows + 9][dz_lds::kXPitch];  // rows t0-8 ..; the last row a spare
  bf16_t dy[dz_lds::kRows + 1][dz_lds::kYPitch];  // the last row a spare
  u32x4_t u[2][RT * KB][64];                       // operand o = m*KB + kb, per lane
};

template <int W, int RT>
__global__ __launch_bounds__(dz_lds::kThreads) void lowrank_dz_lds_kernel(LowrankArgs a) {
  using namespace dz_lds;
  using Sh = DzLdsShared<W, RT>;
  constexpr int WP = Sh::WP, KB = Sh::KB, NOP = RT * KB;
  constexpr int NOW = (NOP + kWaves - 1) / kWaves;     // operands each wave fetches per sub-chunk
  constexpr int PPR = kCh / 8;                          // 16-byte pieces per row and stage
  constexpr int NXC = (kRows + 8) * PPR, NYC = kRows * PPR;  // pieces of x and dy per stage
  constexpr int NXS = (NXC + kThreads - 1) / kThreads, NYS = (NYC + kThreads - 1) / kThreads;
  constexpr int NSL = NXS + NYS;
  __shared__ Sh sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = lane & 15, g = lane >> 4;
  const uint32_t rt = blockIdx.x % a.n_rtile;
  const uint32_t rest = blockIdx.x / a.n_rtile;
  const int64_t cs = rest % a.n_csplit, b = rest / a.n_csplit;
  const int64_t T = a.T, D = a.D, DW = D * W;
  const int R = a.R;
  const int64_t t0 = (int64_t)rt * kRows;
  const int64_t c_begin = cs * a.csplit_len;
  const int64_t c_end = c_begin + a.csplit_len < D ? c_begin + a.csplit_len : D;
  // (rows t0-8 .. t0+kRows-1 of this sequence; offsets stay below 2 GiB as in every
  // matrix-core kernel here)
  const buf_t ub = make_buf(a.U, (uint64_t)(R * DW * 2));
  const buf_t xb = make_buf(static_cast<const bf16_t*>(a.x) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t dyb = make_buf(static_cast<const bf16_t*>(a.dy) + b * T * D, (uint64_t)(T * D * 2));

  // Staging slots with a fixed tensor each (so the buffer resource is uniform): slots
  // 0 .. NXS-1 load x pieces q = tid + kThreads*i (x row q/PPR, i.e. step t0-8+q/PPR,
  // channels 8*(q%PPR) .. of the stage), the last NYS slots dy pieces. Rows outside the
  // sequence and channels past the split read zero; idle lanes write a spare row.
  uint32_t q_off[NSL];  // byte offset of the piece in the stage at channel 0 (kOutOfRange: idle or before 0)
  int q_c[NSL];         // its first channel relative to the stage
  uint32_t q_lds[NSL];  // its place in the shared block
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const bool xs = i < NXS;
    const int q = (int)threadIdx.x + kThreads * (xs ? i : i - NXS);
    const bool on = q < (xs ? NXC : NYC);
    const int row = q / PPR, piece = q % PPR;
    const int64_t t = t0 + (xs ? row - 8 : row);
    q_c[i] = 8 * piece;
    q_off[i] = (on && t >= 0 && t < T) ? (uint32_t)((t * D + 8 * piece) * 2) : kOutOfRange;
    q_lds[i] = (uint32_t)(xs ? (on ? reinterpret_cast<uintptr_t>(&sh.x[row][8 * piece])
                                   : reinterpret_cast<uintptr_t>(&sh.x[kRows + 8][0]))
                             : (on ? reinterpret_cast<uintptr_t>(&sh.dy[row][8 * piece])
                                   : reinterpret_cast<uintptr_t>(&sh.dy[kRows][0]))) -
               (uint32_t)reinterpret_cast<uintptr_t>(&sh);
  }
  u32x4_t pre[NSL];
  auto issue_rows = [&](int64_t c0) {
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      // channels past the split (and past D) read zeros
      const uint32_t off = (c0 + q_c[i] < c_end && q_off[i] != kOutOfRange) ? q_off[i] + (uint32_t)(c0 * 2)
                                                                               : kOutOfRange;
      pre[i] = buf_load16(i < NXS ? xb : dyb, off);
    }
  };
  auto commit_rows = [&]() {
    char* base = reinterpret_cast<char*>(&sh);
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      const u32x4_t v = pre[i];
      if (i < NXS) {
        float* dst = reinterpret_cast<float*>(base + q_lds[i]);
        *reinterpret_cast<float4*>(dst) = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
        *reinterpret_cast<float4*>(dst + 4) = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
      } else {
        *reinterpret_cast<u32x4_t*>(base + q_lds[i]) = v;
      }
    }
  };
  // U operand o = m*KB + kb of the 16-channel sub-chunk at c0 for this lane: rank
  // 16m + tl, columns 8kb.. of this lane group's (channel, tap) pairs
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
  u32x4_t upre[NOW];
  auto issue_ops = [&](int64_t c0) {
#pragma unroll
    for (int i = 0; i < NOW; ++i) {
      const int o = wave + kWaves * i;
      upre[i] = o < NOP ? load_operand(c0, o) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto commit_ops = [&](int slot) {
#pragma unroll
    for (int i = 0; i < NOW; ++i) {
      const int o = wave + kWaves * i;
      if (o < NOP) sh.u[slot][o][lane] = upre[i];
    }
  };

  f32x4_t acc[kMB][RT];
#pragma unroll
  for (int h = 0; h < kMB; ++h)
#pragma unroll
    for (int m = 0; m < RT; ++m) acc[h][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  issue_rows(c_begin);
  issue_ops(c_begin);
  commit_rows();
  commit_ops(0);
  __syncthreads();
  int slot = 0;
  for (int64_t c0 = c_begin; c0 < c_end; c0 += kCh) {
    issue_rows(c0 + kCh);  // the next stage (past the split: zeros)
#pragma unroll
    for (int sub = 0; sub < kCh / 16; ++sub) {
      const int64_t cs0 = c0 + 16 * sub;
      issue_ops(cs0 + 16);  // the next sub-chunk's operands (past the split: zeros)
      if (cs0 < c_end) {    // the same for the whole block
        bf16x8_t uop[RT][KB];
#pragma unroll
        for (int m = 0; m < RT; ++m)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) uop[m][kb] = as_bf16x8(sh.u[slot][m * KB + kb][lane]);
#pragma unroll
        for (int h = 0; h < kMB; ++h) {
          const int row = 16 * kMB * wave + 16 * h + tl;  // this lane's step, relative to t0
          float dyf[4];
          {
            const uint2 v = *reinterpret_cast<const uint2*>(&sh.dy[row][16 * sub + 4 * g]);
            dyf[0] = bf16_lo(v.x); dyf[1] = bf16_hi(v.x); dyf[2] = bf16_lo(v.y); dyf[3] = bf16_hi(v.y);
          }
          float gv[4 * WP];
#pragma unroll
          for (int k = 0; k < W; ++k) {
            const float4 xk = *reinterpret_cast<const float4*>(&sh.x[row + 8 - k][16 * sub + 4 * g]);  // x[t-k]
            gv[0 * WP + k] = dyf[0] * xk.x;
            gv[1 * WP + k] = dyf[1] * xk.y;
            gv[2 * WP + k] = dyf[2] * xk.z;
            gv[3 * WP + k] = dyf[3] * xk.w;
          }
          if constexpr (WP != W) {
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[i * WP + W] = 0.f;
          }
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            bf16x8_t ghi, glo;
            split_hi_lo(gv + 8 * kb, ghi, glo);
#pragma unroll
            for (int m = 0; m < RT; ++m) acc[h][m] = mfma_16x16x32(uop[m][kb], ghi, acc[h][m]);
#pragma unroll
            for (int m = 0; m < RT; ++m) acc[h][m] = mfma_16x16x32(uop[m][kb], glo, acc[h][m]);
          }
        }
      }
      // the other operand slot was last read in the previous sub-chunk, before its barrier
      commit_ops(slot ^ 1);
      if (sub == kCh / 16 - 1) {
        __syncthreads();  // every wave is done with this stage's rows
        commit_rows();
      }
      __syncthreads();
      slot ^= 1;
    }
  }
  // partial dz of this channel split: lane (t, g) holds dz[t, 16m + 4g + i]
  float* dst = a.dz_part + (cs * a.B + b) * T * (int64_t)R;
#pragma unroll
  for (int h = 0; h < kMB; ++h) {
    const int64_t t = t0 + 16 * kMB * wave + 16 * h + tl;
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
