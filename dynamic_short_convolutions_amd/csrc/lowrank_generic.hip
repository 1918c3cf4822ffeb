// Low-rank dynamic short convolution, plain vector-ALU kernels.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", technical
// summary page, section Metodologia, low-rank factorisation, and the
// fused-kernel section): the filter of channel c, tap k at step t is
//   f[b,t,c,k] = sum_r z[b,t,r] * U[r, c*W+k],
// generated in registers and used at once; it is never written to memory.
//
// These kernels serve float32 tensors and every size the matrix-core path
// does not take, on the vector ALUs: the forward and dx build the filters of
// a few consecutive steps per thread from each U load, dz is a product tiled
// through LDS, and the long sums of dz and dU run in double. Each output
// element is finished by one thread in a fixed order, so results are
// reproducible bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace dsc {

struct LrgArgs {
  const void* x;
  const void* z;
  const void* U;
  const int32_t* pos;  // [B, T] positions within packed sequences, or null
  const void* dy;
  void* out;     // y (forward) or dx (backward)
  int64_t B, T, D;
  int R, residual;
  int ngroups;
};

// The thread's 8*W contiguous columns of one U row, 16 bytes per load (the API keeps
// every tensor 16-byte aligned and D a multiple of 4 in fp32, 8 in bf16, so each row
// slice is aligned): u[i*W + k] for channel 8j+i, tap k. With a half group (fp32,
// n4 == 1) the last 4*W columns read as zeros.
template <typename S, int W>
__device__ __forceinline__ void load_ucols(const S* urow, int n4, float (&u)[8 * W]) {
  if constexpr (sizeof(S) == 4) {
#pragma unroll
    for (int q = 0; q < 2 * W; ++q) {
      const float4 v = q < n4 * W ? *reinterpret_cast<const float4*>(urow + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
      u[4 * q] = v.x; u[4 * q + 1] = v.y; u[4 * q + 2] = v.z; u[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < W; ++q) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(urow + 8 * q);
      u[8 * q + 0] = bf16_lo(v.x); u[8 * q + 1] = bf16_hi(v.x);
      u[8 * q + 2] = bf16_lo(v.y); u[8 * q + 3] = bf16_hi(v.y);
      u[8 * q + 4] = bf16_lo(v.z); u[8 * q + 5] = bf16_hi(v.z);
      u[8 * q + 6] = bf16_lo(v.w); u[8 * q + 7] = bf16_hi(v.w);
    }
  }
}

// Filter taps of the thread's 8 channels at one step: f[i][k] for channel 8j+i.
template <typename S, int W>
__device__ __forceinline__ void gen_filter(const S* zrow, const S* U, int64_t D, int R, int j, int n4,
                                           float (&f)[8][W]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int k = 0; k < W; ++k) f[i][k] = 0.f;
  const int64_t cols = D * W;
  for (int r = 0; r < R; ++r) {
    const float zr = load1(zrow + r);
    float u[8 * W];
    load_ucols<S, W>(U + (int64_t)r * cols + (int64_t)8 * j * W, n4, u);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < W; ++k) f[i][k] = fmaf(zr, u[i * W + k], f[i][k]);
  }
}

// Steps per item: a thread builds the filters of its 8 channels for this many consecutive
// steps of one sequence at once (128 taps in registers), so each 16-byte slice of U it
// loads serves all of them; the U loads, 8*W*4 bytes per rank per step, otherwise bound
// these kernels. On MI355X at B=8, T=4096, D=2048, R=32, W=4 in fp32: forward 4.08 ms
// with one step per item, 2.00 ms with 2, 1.19 ms with 4 (2 waves per SIMD; 8 would spill).
#ifndef DSC_LRG_TILE_TAPS
#define DSC_LRG_TILE_TAPS 128
#endif
template <int W>
constexpr int steps_per_item() {
  return DSC_LRG_TILE_TAPS / (8 * W) > 0 ? DSC_LRG_TILE_TAPS / (8 * W) : 1;
}

// Item idx of a launch over (sequence, tile of ST steps, channel group), group fastest.
struct LrgItem {
  int j;        // channel group
  int64_t row;  // first step of the tile, counted over the batch
  int64_t t;    // its step within the sequence
  int nt;       // steps of the tile inside the sequence
};
__device__ __forceinline__ LrgItem lrg_item(const LrgArgs& a, int64_t idx, int ST) {
  const int64_t ntile = (a.T + ST - 1) / ST;
  LrgItem it;
  it.j = (int)(idx % a.ngroups);
  const int64_t tile = idx / a.ngroups, b = tile / ntile;
  it.t = tile % ntile * ST;
  it.row = b * a.T + it.t;
  it.nt = (int)(a.T - it.t < ST ? a.T - it.t : ST);
  return it;
}

// y of one (tile of steps, channel group) item. Per output the operations and their
// order are those of the definition: the filter as a sum over ranks in rank order,
// then the residual and the taps in tap order.
template <typename S, int W>
__device__ __forceinline__ void lowrank_fwd_generic_item(const LrgArgs& a, int64_t idx) {
  constexpr int ST = steps_per_item<W>();
  const LrgItem it = lrg_item(a, idx, ST);
  const int j = it.j;
  const int n4 = (8 * j + 4 < a.D) ? 2 : 1;
  const S* x = static_cast<const S*>(a.x);
  const S* z = static_cast<const S*>(a.z) + it.row * a.R;
  float f[ST][8][W];
#pragma unroll
  for (int q = 0; q < ST; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < W; ++k) f[q][i][k] = 0.f;
  const int64_t cols = a.D * W;
#pragma unroll 2  // two ranks' loads in flight: forward 1.21 -> 1.06 ms at W = 4 (4 ranks: 256 VGPRs)
  for (int r = 0; r < a.R; ++r) {
    float u[8 * W];
    load_ucols<S, W>(static_cast<const S*>(a.U) + (int64_t)r * cols + (int64_t)8 * j * W, n4, u);
#pragma unroll
    for (int q = 0; q < ST; ++q) {
      const float zr = q < it.nt ? load1(z + (int64_t)q * a.R + r) : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < W; ++k) f[q][i][k] = fmaf(zr, u[i * W + k], f[q][i][k]);
    }
  }
#pragma unroll
  for (int q = 0; q < ST; ++q) {
    if (q >= it.nt) continue;
    const int64_t row = it.row + q, t = it.t + q;
    const int p = a.pos ? a.pos[row] : W;  // taps k > p reach into another sequence
    float out[8], xv[8];
    Group8<S>::load(x + row * a.D + 8 * j, xv, n4);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = a.residual ? xv[i] : 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      if (t - k < 0 || (k > 0 && k > p)) break;
      Group8<S>::load(x + (row - k) * a.D + 8 * j, xv, n4);
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = fmaf(f[q][i][k], xv[i], out[i]);
    }
    Group8<S>::store(static_cast<S*>(a.out) + row * a.D + 8 * j, out, n4);
  }
}

// Items of a launch: sequences x tiles of steps x channel groups.
template <int W>
__device__ __host__ __forceinline__ int64_t lrg_items(const LrgArgs& a) {
  constexpr int ST = steps_per_item<W>();
  return a.B * ((a.T + ST - 1) / ST) * a.ngroups;
}

// y, one thread per (tile of steps, channel group) item, grid-stride (the grid is capped).
template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_fwd_generic_kernel(LrgArgs a) {
  const int64_t n = lrg_items<W>(a);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x)
    lowrank_fwd_generic_item<S, W>(a, idx);
}

// dx[s] = residual*dy[s] + sum_k f(s+k)[c,k] * dy[s+k] for a tile of steps s and one
// channel group. The taps f(s+k)[c,k] of each output are built together, rank by rank
// (z of step s+k against U as the forward reads it: the thread's 8*W columns of each
// U row, 16 bytes per load, shared by the tile's outputs), with the same operations
// per tap as one tap at a time.
template <typename S, int W>
__device__ __forceinline__ void lowrank_dx_generic_item(const LrgArgs& a, int64_t idx) {
  constexpr int ST = steps_per_item<W>();
  const LrgItem it = lrg_item(a, idx, ST);
  const int j = it.j;
  const int n4 = (8 * j + 4 < a.D) ? 2 : 1;
  const S* dy = static_cast<const S*>(a.dy);
  const S* z = static_cast<const S*>(a.z);
  // tap k of step s+k exists: inside the sequence and (packed) within its own sequence
  bool on[ST][W];
#pragma unroll
  for (int q = 0; q < ST; ++q)
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const int64_t s = it.t + q;
      on[q][k] = q < it.nt && s + k < a.T && (!a.pos || k == 0 || k <= a.pos[it.row + q + k]);
    }
  float f[ST][8][W];
#pragma unroll
  for (int q = 0; q < ST; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < W; ++k) f[q][i][k] = 0.f;
  const int64_t cols = a.D * W;
#pragma unroll 2  // as in the forward (the fp32 backward 4.33 -> 4.21 ms)
  for (int r = 0; r < a.R; ++r) {
    float u[8 * W];
    load_ucols<S, W>(static_cast<const S*>(a.U) + (int64_t)r * cols + (int64_t)8 * j * W, n4, u);
    // z of the steps the tile's taps come from: it.row + m, m < ST + W - 1
    float zr[ST + W - 1];
#pragma unroll
    for (int m = 0; m < ST + W - 1; ++m) {
      const bool need = m < it.nt + W - 1 && it.t + m < a.T;
      zr[m] = need ? load1(z + (it.row + m) * a.R + r) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < ST; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < W; ++k) f[q][i][k] = fmaf(on[q][k] ? zr[q + k] : 0.f, u[i * W + k], f[q][i][k]);
  }
#pragma unroll
  for (int q = 0; q < ST; ++q) {
    if (q >= it.nt) continue;
    const int64_t row = it.row + q;
    float out[8], dv[8];
    Group8<S>::load(dy + row * a.D + 8 * j, dv, n4);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = a.residual ? dv[i] : 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      if (!on[q][k]) continue;
      Group8<S>::load(dy + (row + k) * a.D + 8 * j, dv, n4);
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = fmaf(f[q][i][k], dv[i], out[i]);
    }
    Group8<S>::store(static_cast<S*>(a.out) + row * a.D + 8 * j, out, n4);
  }
}

template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_dx_generic_kernel(LrgArgs a) {
  const int64_t n = lrg_items<W>(a);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x)
    lowrank_dx_generic_item<S, W>(a, idx);
}

// dz[b,t,r] = sum_{c,k} dy[b,t,c] x[b,t-k,c] U[r,c*W+k], a product of the [tokens, D*W]
// matrix of terms g = dy*x (built on the fly) with U transposed. A block takes a tile of
// 64 tokens x 32 ranks; per chunk of 8 channels it stages g (8*W rows of 64 tokens) and
// U (8*W rows of 32 ranks) in LDS, in double, and each thread adds the products into
// its 2 tokens x 4 ranks. Every output is one thread's running sum over (c, k) in
// order, so results are reproducible bit for bit. The sums are carried in double: the
// terms of these long contractions cancel, and an fp32 running sum loses up to its own
// magnitude times the number of terms times 2^-24, above the fp32 tolerance of a small
// result; the products g are exact in double. (One block per token and 16 ranks, its
// threads striding over channels, had read all of U's chunk for every token: 2.8 ms at
// B=8, T=4096, D=2048, R=32, W=4 in fp32.)
constexpr int kDzTok = 64, kDzRank = 32, kDzCh = 8;
static_assert(kDzTok == 64 && kDzRank == 32, "the thread layout below: 32 token pairs x 8 rank quads");

template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_dz_generic_kernel(LrgArgs a, void* dz) {
  __shared__ __attribute__((aligned(16))) double gs[kDzCh * W][kDzTok];
  __shared__ __attribute__((aligned(16))) double us[kDzCh * W][kDzRank];
  const int tid = threadIdx.x;
  const int tg = tid % 32, rg = tid / 32;  // this thread's tokens 2tg, 2tg+1 and ranks 4rg..4rg+3
  const int r0 = kDzRank * blockIdx.y;
  const int64_t rows = a.B * a.T, ntiles = (rows + kDzTok - 1) / kDzTok;
  const S* x = static_cast<const S*>(a.x);
  const S* dy = static_cast<const S*>(a.dy);
  const S* U = static_cast<const S*>(a.U);
  const int64_t cols = a.D * W;
  // tiles are block-uniform, so every thread takes the barriers below together
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * kDzTok;
    double acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int64_t c0 = 0; c0 < a.D; c0 += kDzCh) {
      // g of the tile's tokens x kDzCh channels: (token, channel) pairs e = tid + 256h
#pragma unroll
      for (int h = 0; h < (kDzTok * kDzCh + 255) / 256; ++h) {
        const int e = tid + 256 * h, m = e / kDzCh, c = e % kDzCh;
        if (m >= kDzTok) continue;
        const int64_t row = row0 + m, ch = c0 + c;
        double g[W];
#pragma unroll
        for (int k = 0; k < W; ++k) g[k] = 0.0;
        if (row < rows && ch < a.D) {
          const int64_t t = row % a.T;
          const int p = a.pos ? a.pos[row] : W;
          const double d = load1(dy + row * a.D + ch);
#pragma unroll
          for (int k = 0; k < W; ++k)
            if (t - k >= 0 && (k == 0 || k <= p)) g[k] = d * (double)load1(x + (row - k) * a.D + ch);
        }
#pragma unroll
        for (int k = 0; k < W; ++k) gs[c * W + k][m] = g[k];
      }
      // U of the tile's ranks x kDzCh channels (all W taps): (rank, channel) pairs
#pragma unroll
      for (int h = 0; h < (kDzRank * kDzCh + 255) / 256; ++h) {
        const int e = tid + 256 * h, r = e / kDzCh, c = e % kDzCh;
        if (r >= kDzRank) continue;
        const int64_t ch = c0 + c;
        const bool in = r0 + r < a.R && ch < a.D;
        const S* u = U + (int64_t)(r0 + r) * cols + ch * W;
#pragma unroll
        for (int k = 0; k < W; ++k) us[c * W + k][r] = in ? (double)load1(u + k) : 0.0;
      }
      __syncthreads();
#pragma unroll 4
      for (int kk = 0; kk < kDzCh * W; ++kk) {
        const double2 gv = *reinterpret_cast<const double2*>(&gs[kk][2 * tg]);
        const double2 u01 = *reinterpret_cast<const double2*>(&us[kk][4 * rg]);
        const double2 u23 = *reinterpret_cast<const double2*>(&us[kk][4 * rg + 2]);
        const double gg[2] = {gv.x, gv.y}, uu[4] = {u01.x, u01.y, u23.x, u23.y};
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fma(gg[i], uu[j], acc[i][j]);
      }
      __syncthreads();  // gs and us are written again by the next chunk
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = row0 + 2 * tg + i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + 4 * rg + j;
        if (row < rows && r < a.R) store1(static_cast<S*>(dz) + row * a.R + r, (float)acc[i][j]);
      }
    }
  }
}

// dU[r, c*W+k] = sum_{b,t} z[b,t,r] dy[b,t,c] x[b,t-k,c], in double (as dz above).
// A block takes 16 channels (all W taps of each) and a chunk of RC ranks; its 256
// threads are the 16 channels times 16 time lanes, lane s summing the steps
// t = s (mod 16) of every sequence in order, so dy and z of a step are loaded once
// for all W x RC sums. The 16 lanes' sums are added in lane order through LDS, one
// rank at a time. (One thread walking every token of one column had left 64 blocks
// on the GPU: 86 ms for the fp32 backward at B=8, T=4096, D=2048, R=32, W=4.)
constexpr int kDUCh = 16, kDULanes = 16;
template <int W>
constexpr int du_ranks() { return W <= 4 ? 16 : 8; }  // the W x RC double sums stay in registers

template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_dU_generic_kernel(LrgArgs a, void* dU) {
  constexpr int RC = du_ranks<W>();
  __shared__ double red[kDULanes][kDUCh * W + 1];
  const int64_t cols = a.D * W, ncb = (a.D + kDUCh - 1) / kDUCh;
  const int cl = (int)(threadIdx.x % kDUCh), s = (int)(threadIdx.x / kDUCh);
  const int r0 = RC * blockIdx.y;
  const S* x = static_cast<const S*>(a.x);
  const S* dy = static_cast<const S*>(a.dy);
  const S* z = static_cast<const S*>(a.z);
  // z ranks r0 .. r0+RC-1 of a row as 16-byte loads where they are aligned and all exist
  const bool zvec = sizeof(S) == 4 && a.R % 4 == 0 && r0 + RC <= a.R;
  // channel blocks strided over the (capped) grid; the loop is uniform over the block
  for (int64_t cb = blockIdx.x; cb < ncb; cb += gridDim.x) {
    const int64_t c = cb * kDUCh + cl;
    double acc[RC][W];
#pragma unroll
    for (int q = 0; q < RC; ++q)
#pragma unroll
      for (int k = 0; k < W; ++k) acc[q][k] = 0.0;
    if (c < a.D) {
      for (int64_t b = 0; b < a.B; ++b) {
        for (int64_t t = s; t < a.T; t += kDULanes) {
          const int64_t row = b * a.T + t;
          const double d = (double)load1(dy + row * a.D + c);
          float zr[RC];
          if (zvec) {
#pragma unroll
            for (int q = 0; q < RC; q += 4) {
              const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(z) + row * a.R + r0 + q);
              zr[q] = v.x; zr[q + 1] = v.y; zr[q + 2] = v.z; zr[q + 3] = v.w;
            }
          } else {
#pragma unroll
            for (int q = 0; q < RC; ++q) zr[q] = r0 + q < a.R ? load1(z + row * a.R + r0 + q) : 0.f;
          }
          const int p = a.pos ? a.pos[row] : W;
#pragma unroll
          for (int k = 0; k < W; ++k) {
            if (t < k || (k > 0 && k > p)) continue;
            const double g = d * (double)load1(x + (row - k) * a.D + c);
#pragma unroll
            for (int q = 0; q < RC; ++q) acc[q][k] = fma((double)zr[q], g, acc[q][k]);
          }
        }
      }
    }
    // the 16 x W outputs of each rank: the 16 lanes added in order
    for (int q = 0; q < RC; ++q) {
#pragma unroll
      for (int k = 0; k < W; ++k) red[s][cl * W + k] = acc[q][k];
      __syncthreads();
      for (int o = (int)threadIdx.x; o < kDUCh * W; o += 256) {
        const int64_t oc = cb * kDUCh + o / W;
        if (oc < a.D && r0 + q < a.R) {
          double v = red[0][o];
#pragma unroll
          for (int l = 1; l < kDULanes; ++l) v += red[l][o];
          store1(static_cast<S*>(dU) + (int64_t)(r0 + q) * cols + oc * W + o % W, (float)v);
        }
      }
      __syncthreads();  // red[] is written again for the next rank
    }
  }
}

namespace {

// Grid-stride launches: at most 2^20 blocks of 256 threads (2^28 work-items, far below
// a dispatch's 32-bit limit), each block looping over the rest.
constexpr int64_t kMaxGenericBlocks = (int64_t)1 << 20;
inline unsigned capped_blocks(int64_t items) {
  const int64_t b = (items + 255) / 256;
  return (unsigned)(b < kMaxGenericBlocks ? b : kMaxGenericBlocks);
}

template <typename S, int W>
hipError_t fwd_generic(const LrgArgs& a, hipStream_t s) {
  const int64_t n = lrg_items<W>(a);
  hipLaunchKernelGGL((lowrank_fwd_generic_kernel<S, W>), dim3(capped_blocks(n)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename S, int W>
hipError_t bwd_generic(const LrgArgs& a, void* dz, void* dU, hipStream_t s) {
  const int64_t n = lrg_items<W>(a);
  hipLaunchKernelGGL((lowrank_dx_generic_kernel<S, W>), dim3(capped_blocks(n)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rchunks = (unsigned)((a.R + kDzRank - 1) / kDzRank);
  const int64_t tiles = (a.B * a.T + kDzTok - 1) / kDzTok;
  const unsigned tile_blocks = (unsigned)(tiles < (int64_t)1 << 16 ? tiles : (int64_t)1 << 16);
  hipLaunchKernelGGL((lowrank_dz_generic_kernel<S, W>), dim3(tile_blocks, rchunks), dim3(256), 0, s, a, dz);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // (at most 2^16 x 16 blocks of 256 threads: 2^28 work-items; the kernel strides over the rest)
  const int64_t ncb = (a.D + kDUCh - 1) / kDUCh;
  const unsigned du_chunks = (unsigned)((a.R + du_ranks<W>() - 1) / du_ranks<W>());
  hipLaunchKernelGGL((lowrank_dU_generic_kernel<S, W>), dim3((unsigned)(ncb < 65536 ? ncb : 65536), du_chunks),
                     dim3(256), 0, s, a, dU);
  return hipGetLastError();
}

template <typename S>
hipError_t fwd_generic_w(const LrgArgs& a, int W, hipStream_t s) {
  switch (W) {
    case 1: return fwd_generic<S, 1>(a, s);
    case 2: return fwd_generic<S, 2>(a, s);
    case 3: return fwd_generic<S, 3>(a, s);
    case 4: return fwd_generic<S, 4>(a, s);
    case 5: return fwd_generic<S, 5>(a, s);
    case 6: return fwd_generic<S, 6>(a, s);
    case 7: return fwd_generic<S, 7>(a, s);
    default: return fwd_generic<S, 8>(a, s);
  }
}

template <typename S>
hipError_t bwd_generic_w(const LrgArgs& a, int W, void* dz, void* dU, hipStream_t s) {
  switch (W) {
    case 1: return bwd_generic<S, 1>(a, dz, dU, s);
    case 2: return bwd_generic<S, 2>(a, dz, dU, s);
    case 3: return bwd_generic<S, 3>(a, dz, dU, s);
    case 4: return bwd_generic<S, 4>(a, dz, dU, s);
    case 5: return bwd_generic<S, 5>(a, dz, dU, s);
    case 6: return bwd_generic<S, 6>(a, dz, dU, s);
    case 7: return bwd_generic<S, 7>(a, dz, dU, s);
    default: return bwd_generic<S, 8>(a, dz, dU, s);
  }
}

LrgArgs make_args(const LowrankProblem& p, void* out) {
  LrgArgs a;
  a.x = p.x; a.z = p.z; a.U = p.U; a.pos = p.pos; a.dy = p.dy; a.out = out;
  a.B = p.B; a.T = p.T; a.D = p.D; a.R = p.R; a.residual = p.residual;
  a.ngroups = (int)((p.D + 7) / 8);
  return a;
}

}  // namespace

hipError_t lowrank_fwd_generic(const LowrankProblem& p, hipStream_t s) {
  const LrgArgs a = make_args(p, p.y);
  return p.bf16 ? fwd_generic_w<bf16_t>(a, p.W, s) : fwd_generic_w<float>(a, p.W, s);
}

hipError_t lowrank_bwd_generic(const LowrankProblem& p, hipStream_t s) {
  const LrgArgs a = make_args(p, p.dx);
  return p.bf16 ? bwd_generic_w<bf16_t>(a, p.W, p.dz, p.dU, s) : bwd_generic_w<float>(a, p.W, p.dz, p.dU, s);
}

}  // namespace dsc
