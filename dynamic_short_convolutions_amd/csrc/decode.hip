// Decode step of the causal dynamic short convolution: one new token per row.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", technical
// summary page, section Metodologia, Mecanismo, taken at a single step t): with
// the filter f[b,c,k] of row b's incoming token,
//   y[b,c] = residual*x[b,c] + sum_{k=0}^{min(W-1,t)} f[b,c,k] * x_{t-k}[c],
// where x_t = x[b,:] and the earlier inputs come from the row's ring
//   state[b, s mod (W-1), :] = x_s,
// after which x[b,:] replaces x_{t-W+1} in slot t mod (W-1). t = pos[b]; a
// negative pos marks an idle row (nothing written for it). Head-wise filters
// are w[b, c/Hc, k]; low-rank filters sum_r z[b,r] U[r, c*W+k] (Parametrizacao
// 1, fused-kernel section), generated in registers.
//
// Every (row, channel) element belongs to exactly one lane, which reads its ring
// slots before it overwrites the oldest one: the in-place ring update needs no
// synchronisation. The whole step is one kernel; its traffic is x, the W-1
// ring slots and the filter read, y and one ring slot written, per row.
#include "launch.hpp"
#include "lowrank_mfma.hpp"

namespace dsc {

struct DecodeArgs {
  const void* x;
  const void* w;
  const void* z;
  const void* U;
  const int32_t* pos;
  void* state;
  void* y;
  int64_t B, D, G;
  int R, residual;
  int64_t Hc;
  // matrix-core low-rank kernel: channel blocks of 64, blocks of 16 rows per
  // workgroup, workgroups per channel block
  int n_cblk, tiles_per_block, n_rgrp;
};

// One 16-byte vector of a row: 8 bf16 or 4 fp32 channels.
template <typename S>
struct Vec16;

template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(u32x4_t q, float (&v)[8]) {
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
  static __device__ __forceinline__ u32x4_t pack(const float (&v)[8]) {
    u32x4_t q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]);
    q.w = pack_bf16x2(v[6], v[7]);
    return q;
  }
};

template <>
struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(u32x4_t q, float (&v)[4]) {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  }
  static __device__ __forceinline__ u32x4_t pack(const float (&v)[4]) {
    u32x4_t q;
    q.x = __float_as_uint(v[0]); q.y = __float_as_uint(v[1]);
    q.z = __float_as_uint(v[2]); q.w = __float_as_uint(v[3]);
    return q;
  }
};

// Row b's ring, all W-1 slots of the vector at channel c0, in slot order. These
// loads do not depend on the row's position, so they are issued together with
// the position itself; each tap then picks its slot.
template <typename S, int W>
__device__ __forceinline__ void load_ring(const DecodeArgs& a, int64_t b, int64_t c0, u32x4_t (&hq)[W > 1 ? W - 1 : 1]) {
  constexpr int NS = W - 1;
  const S* const ring = static_cast<const S*>(a.state) + b * NS * a.D + c0;
  // compile-time indices throughout, so the array lives in registers
  static_for<0, NS>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    hq[j] = *reinterpret_cast<const u32x4_t*>(ring + j * a.D);
  });
}

// Slot (st - k) mod NS of the ring, zero when t < k (a step before the sequence's
// start, whose slot holds no input of this sequence and is never used).
template <int NS, typename V>
__device__ __forceinline__ V ring_tap(const V (&h)[NS > 0 ? NS : 1], int st, int t, int k) {
  const int slot = st - k < 0 ? st - k + NS : st - k;
  V v = h[0];
  static_for<1, NS>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    v = slot == j ? h[j] : v;
  });
  return t >= k ? v : V{};
}

// The convolution of one thread's vector of channels c0 .. c0+N-1 of row b at step
// t >= 0 given its filters f, then the y store and the ring update.
template <typename S, int W>
__device__ __forceinline__ void decode_vector(const DecodeArgs& a, int64_t b, int64_t c0, int t, u32x4_t xq,
                                              const u32x4_t (&hq)[W > 1 ? W - 1 : 1],
                                              const float (&f)[Vec16<S>::N][W]) {
  constexpr int N = Vec16<S>::N;
  constexpr int NS = W - 1;
  const float res = a.residual ? 1.f : 0.f;
  float xv[N], acc[N];
  Vec16<S>::unpack(xq, xv);
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = (f[i][0] + res) * xv[i];
  S* const y = static_cast<S*>(a.y);
  if constexpr (NS > 0) {
    const int st = t % NS;  // slot of x_t, holding x_{t-NS} until the end of this step
#pragma unroll
    for (int k = 1; k <= NS; ++k) {
      float hv[N];
      Vec16<S>::unpack(ring_tap<NS>(hq, st, t, k), hv);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] = fmaf(f[i][k], hv[i], acc[i]);
    }
    *reinterpret_cast<u32x4_t*>(y + b * a.D + c0) = Vec16<S>::pack(acc);
    // after every read of the ring (the loads above)
    *reinterpret_cast<u32x4_t*>(static_cast<S*>(a.state) + (b * NS + st) * a.D + c0) = xq;
  } else {
    *reinterpret_cast<u32x4_t*>(y + b * a.D + c0) = Vec16<S>::pack(acc);
  }
}

// An empty asm statement that reads v. Placed before a branch on the row's
// position, it keeps the loads that produce v above that branch: otherwise the
// compiler sinks them below it, and every load waits for the position first.
template <typename T>
__device__ __forceinline__ void issued_before_branch(const T& v) {
  asm volatile("" ::"v"(v));
}

// W filter taps at p (storage type S) with the widest loads their alignment allows:
// p is a multiple of W elements past a 16-byte aligned base.
template <typename S, int W>
__device__ __forceinline__ void load_taps(const S* p, float (&v)[W]) {
  constexpr int BYTES = W * (int)sizeof(S);
  if constexpr (BYTES % 16 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      float u[16 / sizeof(S)];
      Vec16<S>::unpack(reinterpret_cast<const u32x4_t*>(p)[i], u);
#pragma unroll
      for (int e = 0; e < (int)(16 / sizeof(S)); ++e) v[i * (16 / sizeof(S)) + e] = u[e];
    }
  } else if constexpr (BYTES % 8 == 0 && sizeof(S) == 2) {
#pragma unroll
    for (int i = 0; i < BYTES / 8; ++i) {
      const u32x2_t q = reinterpret_cast<const u32x2_t*>(p)[i];
      v[4 * i + 0] = bf16_lo(q.x); v[4 * i + 1] = bf16_hi(q.x);
      v[4 * i + 2] = bf16_lo(q.y); v[4 * i + 3] = bf16_hi(q.y);
    }
  } else {
#pragma unroll
    for (int k = 0; k < W; ++k) v[k] = load1(p + k);
  }
}

// ----------------------------------------------------------------------------- head-wise

// One thread per (row, 16-byte vector of channels). ONE_HEAD: the vector lies in
// one head (Hc a multiple of the vector width), so its W taps are loaded once.
// Every load is issued before the row's position is known; an idle row stores nothing.
template <typename S, int W, bool ONE_HEAD>
__global__ __launch_bounds__(256) void headwise_decode_kernel(DecodeArgs a) {
  constexpr int N = Vec16<S>::N;
  const int64_t nvec = a.D / N;  // exact: D is a multiple of N
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.B * nvec) return;
  // idx < 2^31 and D < 2^25 (checked by the host): 32-bit divisions
  const int64_t b = (uint32_t)idx / (uint32_t)nvec, c0 = (int64_t)((uint32_t)idx % (uint32_t)nvec) * N;
  const int t = a.pos[b];
  const u32x4_t xq = *reinterpret_cast<const u32x4_t*>(static_cast<const S*>(a.x) + b * a.D + c0);
  u32x4_t hq[W > 1 ? W - 1 : 1];
  if constexpr (W > 1) load_ring<S, W>(a, b, c0, hq);
  const S* const w = static_cast<const S*>(a.w) + b * a.G * W;
  float f[N][W];
  if constexpr (ONE_HEAD) {
    float v[W];
    load_taps<S, W>(w + (uint32_t)c0 / (uint32_t)a.Hc * W, v);
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
      for (int i = 0; i < N; ++i) f[i][k] = v[k];
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) load_taps<S, W>(w + (uint32_t)(c0 + i) / (uint32_t)a.Hc * W, f[i]);
  }
  issued_before_branch(xq);
  static_for<0, W - 1>([&](auto jc) { issued_before_branch(hq[decltype(jc)::value]); });
  static_for<0, W>([&](auto kc) {
    static_for<0, N>([&](auto ic) { issued_before_branch(f[decltype(ic)::value][decltype(kc)::value]); });
  });
  if (t < 0) return;
  decode_vector<S, W>(a, b, c0, t, xq, hq, f);
}

// ----------------------------------------------------------------------------- low-rank, vector ALU

// fp32 tensors and the shapes the matrix-core kernel does not take. One thread per
// (row, vector of N channels): the N*W filter taps of its channels are the
// contiguous columns c0*W .. (c0+N)*W-1 of U, read as W 16-byte vectors per rank.
template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_decode_generic_kernel(DecodeArgs a) {
  constexpr int N = Vec16<S>::N;
  const int64_t nvec = a.D / N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.B * nvec) return;
  const int64_t b = (uint32_t)idx / (uint32_t)nvec, c0 = (int64_t)((uint32_t)idx % (uint32_t)nvec) * N;
  const int t = a.pos[b];
  const u32x4_t xq = *reinterpret_cast<const u32x4_t*>(static_cast<const S*>(a.x) + b * a.D + c0);
  u32x4_t hq[W > 1 ? W - 1 : 1];
  if constexpr (W > 1) load_ring<S, W>(a, b, c0, hq);
  const S* const z = static_cast<const S*>(a.z) + b * a.R;
  const S* const u = static_cast<const S*>(a.U) + c0 * W;
  const int64_t DW = a.D * W;
  float f[N][W];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int k = 0; k < W; ++k) f[i][k] = 0.f;
  for (int r = 0; r < a.R; ++r) {
    const float zr = load1(z + r);
    const S* const ur = u + r * DW;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      float uv[N];
      Vec16<S>::unpack(*reinterpret_cast<const u32x4_t*>(ur + v * N), uv);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const int m = v * N + e;  // column c0*W + m: channel c0 + m/W, tap m%W
        f[m / W][m % W] = fmaf(zr, uv[e], f[m / W][m % W]);
      }
    }
  }
  issued_before_branch(xq);
  static_for<0, W - 1>([&](auto jc) { issued_before_branch(hq[decltype(jc)::value]); });
  if (t < 0) return;
  decode_vector<S, W>(a, b, c0, t, xq, hq, f);
}

// ----------------------------------------------------------------------------- low-rank, matrix cores

// bf16, R a multiple of 8. The filter generation z.U is a [rows x R] by [R x D*W]
// product, computed on the matrix cores: per tap, M = 16 channels of a wave, N = 16
// rows, K = ranks. A workgroup covers 64 channels and a group of blocks of 16 rows;
// it stages the U columns of its channels, [32*KS ranks][64*W columns], in LDS with
// 16-byte loads (ranks past R and columns past D*W read as zero), and each wave
// builds its U^T operands from there once and keeps them in registers over the
// row blocks. Lane l holds row 16*tile + l%16 and channels cw0 + 4*(l/16) .. +3,
// the accumulator layout, so the filters meet the x and ring vectors the lane loads
// without any exchange.
//
// Workgroups of one channel block share its U columns through L2, so they are
// placed on one XCD (workgroups are dealt to the 8 XCDs round robin): workgroup id
// = (cblk/8)*8*n_rgrp + rgrp*8 + cblk%8; ids past the last channel block exit.
template <int W, int KS>
__global__ __launch_bounds__(256) void lowrank_decode_mfma_kernel(DecodeArgs a) {
  constexpr int NS = W - 1;
  constexpr int COLS = 64 * W;     // U columns of the workgroup's 64 channels
  constexpr int PITCH = COLS + 8;  // LDS row pitch (bf16): 16 bytes of padding
  __shared__ __attribute__((aligned(16))) uint16_t ush[32 * KS][PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const uint32_t xcd = blockIdx.x % 8, rest = blockIdx.x / 8;
  const uint32_t rgrp = rest % a.n_rgrp;
  const int cblk = (int)((rest / a.n_rgrp) * 8 + xcd);
  if (cblk >= a.n_cblk) return;  // whole workgroup: before any barrier
  const int64_t B = a.B, D = a.D, DW = D * W;
  const int R = a.R;
  const int64_t cl = (int64_t)cblk * 64 + 16 * wave + 4 * g;  // first of this lane's 4 channels
  const bool lane_ok = cl < D;                                  // D is a multiple of 4
  // Every range is below 2 GiB (checked by the host), so 32-bit offsets address it
  // and kOutOfRange lies beyond all of them: loads there read zero, stores are dropped.
  const buf_t ub = make_buf(a.U, (uint64_t)(R * DW * 2));
  const buf_t xb = make_buf(a.x, (uint64_t)(B * D * 2));
  const buf_t yb = make_buf(a.y, (uint64_t)(B * D * 2));
  const buf_t zb = make_buf(a.z, (uint64_t)(B * R * 2));
  const buf_t pb = make_buf(a.pos, (uint64_t)(B * 4));
  const buf_t sb = make_buf(NS > 0 ? a.state : a.x, (uint64_t)(NS > 0 ? B * NS * D * 2 : 0));

  // U^T operands, built once: the workgroup stages the U columns of its 64 channels
  // in LDS, then each wave reads its A operand of tap k, K step s: row m = channel
  // 16*wave + m of the block, K slot 8*(l/16) + j = rank 32s + 8g + j.
  bf16x8_t ua[W][KS];
  auto stage_u = [&]() {
    // 32*KS rows of COLS/8 16-byte chunks: KS*W chunks per thread, all loads issued
    // before the first LDS write (a loop with a load-to-write chain per trip would
    // wait out one memory latency per chunk)
    constexpr int CHUNKS = COLS / 8, PER = 32 * KS * CHUNKS / 256;
    static_assert(PER * 256 == 32 * KS * CHUNKS, "whole chunks per thread");
    const int64_t col0 = (int64_t)cblk * COLS;
    u32x4_t v[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = tid + 256 * p, r = i / CHUNKS, ch = i % CHUNKS;
      const int64_t col = col0 + ch * 8;  // DW is a multiple of 8: chunks are whole
      v[p] = buf_load16(ub, (r < R && col < DW) ? (uint32_t)((r * DW + col) * 2) : kOutOfRange);
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = tid + 256 * p;
      *reinterpret_cast<u32x4_t*>(&ush[i / CHUNKS][(i % CHUNKS) * 8]) = v[p];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int col = (16 * wave + n) * W + k;
        u32x4_t q;
        uint32_t* qw = reinterpret_cast<uint32_t*>(&q);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 32 * s + 8 * g + 2 * jj;
          qw[jj] = (uint32_t)ush[r][col] | ((uint32_t)ush[r + 1][col] << 16);
        }
        ua[k][s] = as_bf16x8(q);
      }
  };

  const float res = a.residual ? 1.f : 0.f;
  const int ntiles = (int)((B + 15) / 16);
  const int tile0 = (int)rgrp * a.tiles_per_block;
  const int tile1 = tile0 + a.tiles_per_block < ntiles ? tile0 + a.tiles_per_block : ntiles;

  // Each block of 16 rows is loaded whole, position included, before any of it is
  // used: no load waits for the position (every ring slot is read, in slot order).
  // The next block's loads are in flight while one block is computed; blocks past
  // the workgroup's last read nothing and store nothing.
  struct Rows {
    uint32_t pos;
    bf16x8_t z[KS];
    u32x2_t x;
    u32x2_t h[NS > 0 ? NS : 1];
  };
  auto load_rows = [&](int tile, Rows& in) {
    const int64_t b = (int64_t)tile * 16 + n;
    const bool ok = tile < tile1 && b < B;
    const bool v = ok && lane_ok;
    in.pos = __builtin_amdgcn_raw_buffer_load_b32(pb, ok ? (uint32_t)(b * 4) : kOutOfRange, 0, 0);
    load_z<KS>(zb, (int)b, ok, R, g, in.z);
    in.x = buf_load8(xb, v ? (uint32_t)((b * D + cl) * 2) : kOutOfRange);
#pragma unroll
    for (int j = 0; j < NS; ++j) in.h[j] = buf_load8(sb, v ? (uint32_t)(((b * NS + j) * D + cl) * 2) : kOutOfRange);
  };
  auto compute_rows = [&](int tile, const Rows& in) {
    const int64_t b = (int64_t)tile * 16 + n;
    const bool ok = tile < tile1 && b < B;
    const int t = ok ? (int)in.pos : -1;
    const bool st_ok = t >= 0 && lane_ok;
    f32x4_t f[W];
#pragma unroll
    for (int k = 0; k < W; ++k) {
      // the residual rides on tap 0's accumulator: (f_0 + residual) * x
      f[k] = k == 0 ? f32x4_t{res, res, res, res} : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) f[k] = mfma_16x16x32(ua[k][s], in.z[s], f[k]);
    }
    float out[4], xf[4];
    const uint32_t xw[2] = {in.x.x, in.x.y};
    unpack_row<2>(xw, xf);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = f[0][i] * xf[i];
    int st = 0;  // slot of x_t
    if constexpr (NS > 0) st = t >= 0 ? t % NS : 0;
#pragma unroll
    for (int k = 1; k <= NS; ++k) {
      const u32x2_t hk = ring_tap<NS>(in.h, st, t, k);
      const uint32_t hw[2] = {hk.x, hk.y};
      float hf[4];
      unpack_row<2>(hw, hf);
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = fmaf(f[k][i], hf[i], out[i]);
    }
    store_row<2, false>(yb, st_ok ? (uint32_t)((b * D + cl) * 2) : kOutOfRange, out);
    if constexpr (NS > 0) {
      // x_t into the slot of x_{t-NS}, which this lane has read
      buf_store8<false>(sb, st_ok ? (uint32_t)(((b * NS + st) * D + cl) * 2) : kOutOfRange, in.x);
    }
  };

  Rows ra, rb;
  load_rows(tile0, ra);  // in flight during the U staging
  stage_u();
  for (int tile = tile0; tile < tile1; tile += 2) {
    load_rows(tile + 1, rb);
    compute_rows(tile, ra);
    load_rows(tile + 2, ra);
    compute_rows(tile + 1, rb);
  }
}

// ----------------------------------------------------------------------------- ring from a prompt

// One thread per (row, one of the W-1 last prompt steps, 16-byte vector): copies
// x[b, s, vector] into slot s mod (W-1), s = n-1-j for n = clamp(len[b], 0, T).
struct PrefillArgs {
  const void* x;
  const int32_t* len;
  void* state;
  int64_t B, T, nvec;  // nvec: 16-byte vectors per row
  int NS;
};

__global__ __launch_bounds__(256) void decode_state_from_prefill_kernel(PrefillArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.B * a.NS * a.nvec) return;
  const int64_t v = idx % a.nvec, rest = idx / a.nvec;
  const int j = (int)(rest % a.NS);
  const int64_t b = rest / a.NS;
  int64_t nb = a.len[b];
  nb = nb < 0 ? 0 : (nb > a.T ? a.T : nb);
  const int64_t s = nb - 1 - j;
  if (s < 0) return;
  const u32x4_t* src = static_cast<const u32x4_t*>(a.x) + (b * a.T + s) * a.nvec + v;
  u32x4_t* dst = static_cast<u32x4_t*>(a.state) + (b * a.NS + s % a.NS) * a.nvec + v;
  *dst = *src;
}

// ----------------------------------------------------------------------------- launch

namespace {

DecodeArgs make_args(const DecodeProblem& p) {
  DecodeArgs a{};
  a.x = p.x; a.w = p.w; a.z = p.z; a.U = p.U; a.pos = p.pos; a.state = p.state; a.y = p.y;
  a.B = p.B; a.D = p.D; a.G = p.G; a.R = p.R; a.residual = p.residual;
  a.Hc = p.G > 0 ? p.D / p.G : 0;
  return a;
}

unsigned vector_blocks(const DecodeProblem& p) {
  const int64_t n = p.B * (p.D / (p.bf16 ? 8 : 4));
  return (unsigned)((n + 255) / 256);
}

template <typename S, int W>
hipError_t headwise_launch(const DecodeArgs& a, unsigned blocks, hipStream_t s) {
  if (a.Hc % Vec16<S>::N == 0)
    hipLaunchKernelGGL((headwise_decode_kernel<S, W, true>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((headwise_decode_kernel<S, W, false>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename S>
hipError_t headwise_launch_w(const DecodeArgs& a, int W, unsigned blocks, hipStream_t s) {
  switch (W) {
    case 1: return headwise_launch<S, 1>(a, blocks, s);
    case 2: return headwise_launch<S, 2>(a, blocks, s);
    case 3: return headwise_launch<S, 3>(a, blocks, s);
    case 4: return headwise_launch<S, 4>(a, blocks, s);
    case 5: return headwise_launch<S, 5>(a, blocks, s);
    case 6: return headwise_launch<S, 6>(a, blocks, s);
    case 7: return headwise_launch<S, 7>(a, blocks, s);
    default: return headwise_launch<S, 8>(a, blocks, s);
  }
}

template <typename S, int W>
hipError_t generic_launch(const DecodeArgs& a, unsigned blocks, hipStream_t s) {
  hipLaunchKernelGGL((lowrank_decode_generic_kernel<S, W>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename S>
hipError_t generic_launch_w(const DecodeArgs& a, int W, unsigned blocks, hipStream_t s) {
  switch (W) {
    case 1: return generic_launch<S, 1>(a, blocks, s);
    case 2: return generic_launch<S, 2>(a, blocks, s);
    case 3: return generic_launch<S, 3>(a, blocks, s);
    case 4: return generic_launch<S, 4>(a, blocks, s);
    case 5: return generic_launch<S, 5>(a, blocks, s);
    case 6: return generic_launch<S, 6>(a, blocks, s);
    case 7: return generic_launch<S, 7>(a, blocks, s);
    default: return generic_launch<S, 8>(a, blocks, s);
  }
}

template <int W, int KS>
hipError_t mfma_launch(DecodeArgs a, hipStream_t s) {
  a.n_cblk = (int)((a.D + 63) / 64);
  const int64_t ntiles = (a.B + 15) / 16;
  // Blocks of 16 rows per workgroup: enough workgroups for two per CU (a workgroup
  // keeps one block of rows in flight while it computes another, so the loads in
  // flight grow with the workgroups resident), and at most 8 blocks, so that its U
  // staging is amortised while large batches still spread over many workgroups.
  const int64_t per = a.n_cblk * ntiles / 512;
  a.tiles_per_block = (int)(per < 1 ? 1 : (per > 8 ? 8 : per));
  a.n_rgrp = (int)((ntiles + a.tiles_per_block - 1) / a.tiles_per_block);
  const int64_t blocks = (int64_t)((a.n_cblk + 7) / 8) * 8 * a.n_rgrp;
  hipLaunchKernelGGL((lowrank_decode_mfma_kernel<W, KS>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int W>
hipError_t mfma_launch_ks(const DecodeArgs& a, hipStream_t s) {
  switch ((a.R + 31) / 32) {
    case 1: return mfma_launch<W, 1>(a, s);
    case 2: return mfma_launch<W, 2>(a, s);
    case 3: return mfma_launch<W, 3>(a, s);
    default: return mfma_launch<W, 4>(a, s);
  }
}

hipError_t mfma_launch_w(const DecodeArgs& a, int W, hipStream_t s) {
  switch (W) {
    case 1: return mfma_launch_ks<1>(a, s);
    case 2: return mfma_launch_ks<2>(a, s);
    case 3: return mfma_launch_ks<3>(a, s);
    case 4: return mfma_launch_ks<4>(a, s);
    case 5: return mfma_launch_ks<5>(a, s);
    case 6: return mfma_launch_ks<6>(a, s);
    case 7: return mfma_launch_ks<7>(a, s);
    default: return mfma_launch_ks<8>(a, s);
  }
}

}  // namespace

// Matrix-core path: bf16, R a multiple of 8 (whole 16-byte z vectors), and every
// tensor it addresses through a buffer resource below 2 GiB.
bool lowrank_decode_uses_mfma(int64_t B, int64_t D, int R, int W, bool bf16) {
  const int64_t lim = 0x7fffffff;
  return bf16 && R % 8 == 0 && R >= 8 && R <= 128 && D % 8 == 0 && B * D * 2 < lim &&
         B * (W - 1) * D * 2 < lim && B * R * 2 < lim && (int64_t)R * D * W * 2 < lim;
}

hipError_t headwise_decode(const DecodeProblem& p, hipStream_t s) {
  const DecodeArgs a = make_args(p);
  const unsigned blocks = vector_blocks(p);
  return p.bf16 ? headwise_launch_w<bf16_t>(a, p.W, blocks, s) : headwise_launch_w<float>(a, p.W, blocks, s);
}

hipError_t lowrank_decode(const DecodeProblem& p, hipStream_t s) {
  const DecodeArgs a = make_args(p);
  if (lowrank_decode_uses_mfma(p.B, p.D, p.R, p.W, p.bf16)) return mfma_launch_w(a, p.W, s);
  const unsigned blocks = vector_blocks(p);
  return p.bf16 ? generic_launch_w<bf16_t>(a, p.W, blocks, s) : generic_launch_w<float>(a, p.W, blocks, s);
}

hipError_t decode_state_from_prefill(const PrefillStateProblem& p, hipStream_t s) {
  PrefillArgs a{};
  a.x = p.x; a.len = p.len; a.state = p.state;
  a.B = p.B; a.T = p.T; a.nvec = p.D / (p.bf16 ? 8 : 4); a.NS = p.W - 1;
  const int64_t n = a.B * a.NS * a.nvec;
  hipLaunchKernelGGL(decode_state_from_prefill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsc
