// Head-wise forward with the filters generated from the hidden state in the same
// kernel ("Dynamic Short Convolutions Improve Transformers", technical summary
// page, section Metodologia: the filter of step t is a learned linear map of the
// current hidden state, Parametrizacao, tied across the Hc channels of a head):
//   w[b,t,g,k] = sum_j h[b,t,j] * Wg[g*W+k, j]      (Wg: a linear layer's weight, [G*W, K])
//   y[b,t,c]   = residual*x[b,t,c] + sum_k w[b,t,c/Hc,k] * x[b,t-k,c]
// The filters live only in registers and LDS: they never reach HBM.
//
// A workgroup owns M steps of one sequence (M = 256 for W <= 4, else 128) and 32
// heads (32*W filter columns). Its four waves each form MW = M/4 rows of the
// filter tile, all 32*W columns, on the matrix cores (v_mfma_f32_16x16x32_bf16;
// A = hidden-state rows, B = generator rows, both K-contiguous). The K loop runs
// in stages of 64 values through one LDS buffer: the next stage is loaded into
// registers while the current one is multiplied, then written to LDS between two
// barriers. The epilogue writes the fp32 filters of half the tile to LDS at a time
// (waves 0-1, then 2-3) and the whole workgroup convolves those M/2 steps over its
// 32*Hc channels, in units of 8 channels by 8 steps whose W-1+8 input rows are
// loaded at once. Workgroups are ordered so that an XCD runs 4 step tiles against
// every head block in turn, sharing the hidden-state rows in its L2.
// With packed sequences (POS) tap k of step t applies only if k <= pos[b,t]; the
// masks are selects, so nothing of one sequence reaches another.
#include "headwise_kernels.hpp"
#include "launch.hpp"
#include "lowrank_mfma.hpp"

namespace dsc {

struct GenArgs {
  const void* x;
  const void* h;
  const void* Wg;
  const int32_t* pos;  // [B, T] with POS
  void* y;             // y (forward) or dx (backward)
  const void* dy;      // backward
  void* dw;            // backward
  int64_t B, T, D, K;
  int G, Hc, residual;
  int n_gblk;   // head blocks of 32 heads
  int ntps;     // step tiles per sequence
  int n_tt;     // step tiles in all
  int groups;   // groups of 4 step tiles per XCD
};

constexpr int kGenKS = 64;   // K values per stage
constexpr int kGenCS = 8;    // steps per convolution unit

template <int W>
constexpr int gen_mw() { return W <= 4 ? 64 : 32; }  // filter rows per wave
template <int W>
constexpr int gen_m() { return 4 * gen_mw<W>(); }     // steps per workgroup

// Staged rows are 64 K-values (128 bytes, eight 16-byte chunks) with no padding;
// chunk c of row r sits at chunk position c ^ (r % 8). Eight lanes that read one
// chunk index from eight consecutive rows, or eight chunks of one row, then touch
// eight distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ (row & 7)) * 8; }

__device__ __forceinline__ void unpack8(u32x4_t q, float (&v)[8]) {
  v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
  v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
  v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}

// One K stage of the operands, or (epilogue) the fp32 filters of ROWS steps:
// row = step, head g's W taps at g*W .. g*W+W-1, row pitch a multiple of 16 bytes.
template <int W, int M, int ROWS>
union GenSharedT {
  struct {
    uint16_t a[M][kGenKS];       // hidden-state rows
    uint16_t b[32 * W][kGenKS];  // generator rows
  } g;
  float wt[ROWS][32 * W + 4];
};
// the forward's epilogue holds half the tile's steps
template <int W>
using GenShared = GenSharedT<W, gen_m<W>(), gen_m<W>() / 2>;

// The filter tile of one workgroup on the matrix cores: rows t0 .. t0+M-1 (M = 4*MW)
// of sequence b (rows past T are zero), the 32*W columns of head block gblk. On return
// acc[mt][nt] holds, in accumulator i, row MW*wave + 16*mt + 4*(lane/16) + i, column
// 16*nt + lane%16.
template <int W, int MW, typename SH>
__device__ __forceinline__ void gen_filter_tile(const GenArgs& a, SH& sh, int64_t b, int t0, int gblk,
                                                f32x4_t (&acc)[MW / 16][2 * W]) {
  constexpr int M = 4 * MW;
  constexpr int MTL = MW / 16;   // MFMA row tiles per wave
  constexpr int NT = 32 * W;     // filter columns of the workgroup
  constexpr int NTL = NT / 16;   // MFMA column tiles
  constexpr int APER = M * kGenKS / 8 / 256;   // 16-byte chunks per thread and stage
  constexpr int BPER = NT * kGenKS / 8 / 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t T = a.T, K = a.K;
  // per-sequence ranges below 2 GiB (checked by the host): rows past T read zero
  const buf_t hb = make_buf(static_cast<const bf16_t*>(a.h) + b * T * K, (uint64_t)(T * K * 2));
  const buf_t wb = make_buf(static_cast<const bf16_t*>(a.Wg) + (int64_t)gblk * NT * K, (uint64_t)(NT * K * 2));
  // each thread's chunks: byte offsets in stage 0 (rows past T start out of range,
  // and stay there: kOutOfRange + a stage offset is still past every resource)
  uint32_t aoff[APER], boff[BPER];
#pragma unroll
  for (int p = 0; p < APER; ++p) {
    const int c = tid + 256 * p, t = t0 + (c >> 3);
    aoff[p] = t < T ? (uint32_t)(((int64_t)t * K + (c & 7) * 8) * 2) : kOutOfRange;
  }
#pragma unroll
  for (int p = 0; p < BPER; ++p) {
    const int c = tid + 256 * p;
    boff[p] = (uint32_t)(((int64_t)(c >> 3) * K + (c & 7) * 8) * 2);
  }
  const int nks = (int)(K / kGenKS);
  u32x4_t ra[APER], rb[BPER];
  // stages past the last one read out of range: zeros, and no memory traffic
  auto load_stage = [&](int ks) {
    const bool live = ks < nks;
    const uint32_t ko = (uint32_t)(ks * kGenKS * 2);
#pragma unroll
    for (int p = 0; p < APER; ++p) ra[p] = buf_load16(hb, live ? aoff[p] + ko : kOutOfRange);
#pragma unroll
    for (int p = 0; p < BPER; ++p) rb[p] = buf_load16(wb, live ? boff[p] + ko : kOutOfRange);
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int p = 0; p < APER; ++p) {
      const int c = tid + 256 * p;
      *reinterpret_cast<u32x4_t*>(&sh.g.a[c >> 3][swz(c >> 3, c & 7)]) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < BPER; ++p) {
      const int c = tid + 256 * p;
      *reinterpret_cast<u32x4_t*>(&sh.g.b[c >> 3][swz(c >> 3, c & 7)]) = rb[p];
    }
  };

#pragma unroll
  for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  load_stage(0);
  store_stage();
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    load_stage(ks + 1);                 // in flight while this stage is multiplied
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
#pragma unroll
    for (int sub = 0; sub < kGenKS / 32; ++sub) {
      // wave: rows MW*wave .. +MW-1, all NT columns
      bf16x8_t av[MTL];
#pragma unroll
      for (int mt = 0; mt < MTL; ++mt)
        av[mt] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&sh.g.a[MW * wave + 16 * mt + l16][swz(l16, 4 * sub + g)]));
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        const bf16x8_t bv = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&sh.g.b[16 * nt + l16][swz(l16, 4 * sub + g)]));
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt) acc[mt][nt] = mfma_16x16x32(av[mt], bv, acc[mt][nt]);
      }
    }
    __syncthreads();  // every wave is done reading the stage
    store_stage();
    __syncthreads();
  }

}

template <int W, bool POS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gen_fwd_kernel(GenArgs a) {
  constexpr int MW = gen_mw<W>();
  constexpr int M = gen_m<W>();
  constexpr int MTL = MW / 16;   // MFMA row tiles per wave
  constexpr int NTL = 2 * W;     // MFMA column tiles (32*W filter columns)
  __shared__ __attribute__((aligned(16))) GenShared<W> sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const uint32_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const uint32_t grp = local / (4 * a.n_gblk), rr = local % (4 * a.n_gblk);
  const int gblk = (int)(rr / 4);
  const int tt = (int)((grp * 4 + rr % 4) * 8 + xcd);
  if (tt >= a.n_tt) return;  // whole workgroup, before any barrier
  const int64_t b = tt / a.ntps;
  const int t0 = (tt % a.ntps) * M;
  const int64_t T = a.T, D = a.D;

  f32x4_t acc[MTL][NTL];
  gen_filter_tile<W, MW>(a, sh, b, t0, gblk, acc);

  // ---------------------------------------------------------------- convolution
  // units: (channel group of 8, slice of kGenCS steps); a group lies in one head (Hc % 8 == 0)
  const int ngr = 4 * a.Hc;  // 32 heads * Hc channels / 8
  const int64_t cbase = (int64_t)gblk * 32 * a.Hc;
  const buf_t xb = make_buf(static_cast<const bf16_t*>(a.x) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t yb = make_buf(static_cast<bf16_t*>(a.y) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t pb = make_buf(POS ? a.pos + b * T : nullptr, POS ? (uint64_t)(T * 4) : 0);
  const float res = a.residual ? 1.f : 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // accumulator i of tile (mt, nt): row MW*wave + 16*mt + 4*g + i, column 16*nt + l16
    if ((wave >> 1) == half) {
#pragma unroll
      for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sh.wt[MW * (wave & 1) + 16 * mt + 4 * g + i][16 * nt + l16] = acc[mt][nt][i];
    }
    __syncthreads();
    const int th = t0 + half * (M / 2);
    for (int u = tid; u < ngr * (M / 2 / kGenCS); u += 256) {
      const int gi = u % ngr, sl = u / ngr;
      const int head = gi * 8 / a.Hc;
      const uint32_t c0 = (uint32_t)(cbase + 8 * gi);
      const int ts = th + kGenCS * sl;
      if (ts >= T) continue;
      // rows ts-W+1 .. ts+kGenCS-1 at once: rows before 0 are the causal zeros, rows
      // past T lie past the buffer and read zero too. The rows no other unit reads
      // (neither this unit's halo nor the next unit's) are loaded non-temporal, so
      // that they leave the shared rows in L2 (2% faster on the QKV layer).
      constexpr int NR = W - 1 + kGenCS;
      u32x4_t xv[NR];
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int r = ts - (W - 1) + j;
        const uint32_t off = r >= 0 ? (uint32_t)(((int64_t)r * D + c0) * 2) : kOutOfRange;
        if (j >= W - 1 && j < NR - (W - 1)) xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xb, (int)off, 0, 2);
        else xv[j] = buf_load16(xb, off);
      }
      int pv[kGenCS];  // positions of the unit's steps (POS; steps past T read 0, unused)
      if constexpr (POS) {
#pragma unroll
        for (int q = 0; q < kGenCS / 4; ++q) {
          const u32x4_t v = buf_load16(pb, (uint32_t)((ts + 4 * q) * 4));
          pv[4 * q] = (int)v.x; pv[4 * q + 1] = (int)v.y; pv[4 * q + 2] = (int)v.z; pv[4 * q + 3] = (int)v.w;
        }
      }
      float win[W][8];  // before step ts: win[k] = x[ts-1-k]; then shifted per step
#pragma unroll
      for (int k = 0; k < W - 1; ++k) unpack8(xv[W - 2 - k], win[k]);
#pragma unroll
      for (int s = 0; s < kGenCS; ++s) {
        const int t = ts + s;
#pragma unroll
        for (int k = W - 1; k > 0; --k)
#pragma unroll
          for (int i = 0; i < 8; ++i) win[k][i] = win[k - 1][i];
        unpack8(xv[W - 1 + s], win[0]);  // win[k] = x[t-k]
        const float* wrow = &sh.wt[t - th][head * W];
        float out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = res * win[0][i];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const float f = wrow[k];
          if (POS && k > 0) {
            const bool on = k <= pv[s];  // tap k reaches back into this step's own sequence
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = fmaf(on ? f : 0.f, on ? win[k][i] : 0.f, out[i]);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = fmaf(f, win[k][i], out[i]);
          }
        }
        store_row<4, true>(yb, t < T ? (uint32_t)(((int64_t)t * D + c0) * 2) : kOutOfRange, out);
      }
    }
    if (half == 0) __syncthreads();  // the second half overwrites the filters
  }
}

// ----------------------------------------------------------------------------- backward
// The backward of the forward above with respect to x and to the generated filters
// (the chain rule; the page trains with the generator but prints no gradients):
//   dx[b,s,c]   = residual*dy[b,s,c] + sum_k w[b,s+k,c/Hc,k] * dy[b,s+k,c]   (s+k < T)
//   dw[b,t,g,k] = sum_{c in head g} dy[b,t,c] * x[b,t-k,c]
// dx reads the filters of steps s .. s+W-1, which are regenerated here on the matrix
// cores exactly as in the forward and never reach HBM; dw does not involve them
// (the gradients of h and Wg are dw's products with Wg and with h).
//
// A workgroup regenerates the filters of M steps, t0 .. t0+M-1, but writes dx and dw
// only for the first MS = M-W+1 of them: the dx of its last steps needs the next
// W-1 filter rows, so consecutive step tiles overlap by W-1 rows (2.4% more matrix
// work at M = 128, W = 4). M is half the forward's (128 for W <= 4, else 64): the
// accumulators stay live through the first half's convolution next to its x and dy
// rows, and the forward's tile would not fit in the registers. The epilogue holds the fp32 filters of half the tile plus
// the W-1 rows after it in LDS, and convolves in units of 8 channels (of one head)
// by CS steps (8, or 4 for W > 4) whose x rows t-W+1 .. and dy rows .. t+W-1 are
// loaded at once. A head
// of Hc = 8P channels spans P consecutive units; its dw sums are finished across
// their lanes with DPP moves (P a power of two up to 16).
template <int W>
constexpr int gen_bwd_mw() { return W <= 4 ? 32 : 16; }  // filter rows per wave
template <int W>
constexpr int gen_bwd_cs() { return W <= 4 ? 8 : 4; }    // steps per convolution unit

template <int W, int P, bool POS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gen_bwd_kernel(GenArgs a) {
  constexpr int MW = gen_bwd_mw<W>();
  constexpr int M = 4 * MW;
  constexpr int MS = M - (W - 1);       // output steps per workgroup
  constexpr int HR = M / 2 + W - 1;     // filter rows held per half
  constexpr int MTL = MW / 16;
  constexpr int NTL = 2 * W;
  constexpr int CS = gen_bwd_cs<W>();
  __shared__ __attribute__((aligned(16))) GenSharedT<W, M, HR> sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const uint32_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const uint32_t grp = local / (4 * a.n_gblk), rr = local % (4 * a.n_gblk);
  const int gblk = (int)(rr / 4);
  const int tt = (int)((grp * 4 + rr % 4) * 8 + xcd);
  if (tt >= a.n_tt) return;  // whole workgroup, before any barrier
  const int64_t b = tt / a.ntps;
  const int t0 = (tt % a.ntps) * MS;
  const int64_t T = a.T, D = a.D;
  const int G = a.G;

  f32x4_t acc[MTL][NTL];
  gen_filter_tile<W, MW>(a, sh, b, t0, gblk, acc);

  const int ngr = 4 * a.Hc;  // 32 heads * Hc channels / 8
  const int64_t cbase = (int64_t)gblk * 32 * a.Hc;
  const buf_t xb = make_buf(static_cast<const bf16_t*>(a.x) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t dyb = make_buf(static_cast<const bf16_t*>(a.dy) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t dxb = make_buf(static_cast<bf16_t*>(a.y) + b * T * D, (uint64_t)(T * D * 2));
  const buf_t pb = make_buf(POS ? a.pos + b * T : nullptr, POS ? (uint64_t)(T * 4) : 0);
  bf16_t* dws = static_cast<bf16_t*>(a.dw) + (b * T * G + (int64_t)gblk * 32) * W;
  const float res = a.residual ? 1.f : 0.f;
  const int tend = (int)(t0 + MS < T ? t0 + MS : T);  // one past this workgroup's last output step
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // filter rows r0 .. r0+HR-1 of the tile (those below M), from the waves that hold them
    const int r0 = half * (M / 2);
#pragma unroll
    for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = MW * wave + 16 * mt + 4 * g + i;
        if (row >= r0 && row < r0 + HR && row < M) {
#pragma unroll
          for (int nt = 0; nt < NTL; ++nt) sh.wt[row - r0][16 * nt + l16] = acc[mt][nt][i];
        }
      }
    __syncthreads();
    const int th = t0 + r0;
    const int te = th + M / 2 < tend ? th + M / 2 : tend;
    for (int u = tid; u < ngr * (M / 2 / CS); u += 256) {
      const int gi = u % ngr, sl = u / ngr;
      const int head = gi / P, jh = gi % P;
      const uint32_t c0 = (uint32_t)(cbase + 8 * gi);
      const int ts = th + CS * sl;
      if (ts >= te) continue;  // the head's P lanes share ts
      constexpr int NR = W - 1 + CS;
      // x rows ts-W+1 .. ts+CS-1 (before 0: the causal zeros), dy rows ts .. ts+CS+W-2 (past T: zero)
      u32x4_t xv[NR], dv[NR];
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int r = ts - (W - 1) + j;
        xv[j] = buf_load16(xb, r >= 0 && r < T ? (uint32_t)(((int64_t)r * D + c0) * 2) : kOutOfRange);
        dv[j] = buf_load16(dyb, ts + j < T ? (uint32_t)(((int64_t)(ts + j) * D + c0) * 2) : kOutOfRange);
      }
      int pv[NR];  // positions of steps ts .. ts+NR-1 (POS; past T: 0, unused)
      if constexpr (POS) {
#pragma unroll
        for (int j = 0; j < NR; ++j) pv[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(pb, (uint32_t)((ts + j) * 4), 0, 0);
      }
#pragma unroll
      for (int s = 0; s < CS; ++s) {
        const int t = ts + s;
        float dyf[8];
        unpack8(dv[s], dyf);
        // dw: the head's sum over its channels (all P lanes take part in the butterfly)
        float gw[W];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          float xk[8];
          unpack8(xv[W - 1 + s - k], xk);  // x[t-k]
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) sum = fmaf(dyf[i], xk[i], sum);
          sum = head_sum<P>(sum);
          gw[k] = (!POS || k == 0 || k <= pv[s]) ? sum : 0.f;
        }
        // dx: the taps of steps t .. t+W-1 that reach back to t
        float out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = res * dyf[i];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const float f = sh.wt[t + k - th][head * W + k];
          const bool on = !POS || k == 0 || k <= pv[s + k];
          float dk[8];
          unpack8(dv[s + k], dk);
#pragma unroll
          for (int i = 0; i < 8; ++i) out[i] = fmaf(on ? f : 0.f, on ? dk[i] : 0.f, out[i]);
        }
        if (t < te) {
          store_row<4, true>(dxb, (uint32_t)(((int64_t)t * D + c0) * 2), out);
          if (jh == 0) Taps<bf16_t, W>::store(dws + ((int64_t)t * G + head) * W, gw);
        }
      }
    }
    if (half == 0) __syncthreads();  // the second half overwrites the filters
  }
}

namespace {

template <int W, bool POS>
hipError_t gen_launch(GenArgs a, hipStream_t s) {
  constexpr int M = gen_m<W>();
  a.ntps = (int)((a.T + M - 1) / M);
  a.n_tt = (int)(a.B * a.ntps);
  a.groups = (int)(((a.n_tt + 7) / 8 + 3) / 4);
  const int64_t blocks = (int64_t)8 * a.groups * 4 * a.n_gblk;
  hipLaunchKernelGGL((gen_fwd_kernel<W, POS>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int W, int P, bool POS>
hipError_t gen_bwd_launch(GenArgs a, hipStream_t s) {
  constexpr int MS = 4 * gen_bwd_mw<W>() - (W - 1);
  a.ntps = (int)((a.T + MS - 1) / MS);
  a.n_tt = (int)(a.B * a.ntps);
  a.groups = (int)(((a.n_tt + 7) / 8 + 3) / 4);
  const int64_t blocks = (int64_t)8 * a.groups * 4 * a.n_gblk;
  hipLaunchKernelGGL((gen_bwd_kernel<W, P, POS>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int W, bool POS>
hipError_t gen_bwd_by_p(const GenArgs& a, hipStream_t s) {
  switch (a.Hc / 8) {
    case 1: return gen_bwd_launch<W, 1, POS>(a, s);
    case 2: return gen_bwd_launch<W, 2, POS>(a, s);
    case 4: return gen_bwd_launch<W, 4, POS>(a, s);
    case 8: return gen_bwd_launch<W, 8, POS>(a, s);
    case 16: return gen_bwd_launch<W, 16, POS>(a, s);
    default: return hipErrorNotSupported;  // refused by gen_bwd_supported
  }
}

template <bool POS>
hipError_t gen_bwd_by_w(const GenArgs& a, int W, hipStream_t s) {
  switch (W) {
    case 1: return gen_bwd_by_p<1, POS>(a, s);
    case 2: return gen_bwd_by_p<2, POS>(a, s);
    case 3: return gen_bwd_by_p<3, POS>(a, s);
    case 4: return gen_bwd_by_p<4, POS>(a, s);
    case 5: return gen_bwd_by_p<5, POS>(a, s);
    case 6: return gen_bwd_by_p<6, POS>(a, s);
    case 7: return gen_bwd_by_p<7, POS>(a, s);
    default: return gen_bwd_by_p<8, POS>(a, s);
  }
}

}  // namespace

bool gen_bwd_supported(int64_t B, int64_t T, int64_t D, int64_t G, int W, int64_t K) {
  if (!gen_fwd_supported(B, T, D, G, W, K)) return false;
  const int64_t P = D / G / 8;  // units per head: a power of two up to 16
  if (P < 1 || P > 16 || (P & (P - 1)) != 0) return false;
  // the grid at the smallest output step tile (64 - 7)
  const int64_t n_tt = B * ((T + 56) / 57);
  const int64_t groups = ((n_tt + 7) / 8 + 3) / 4;
  return (int64_t)8 * groups * 4 * (G / 32) < 0x7fffffff;
}

hipError_t headwise_bwd_gen(const GenProblem& p, hipStream_t s) {
  GenArgs a{};
  a.x = p.x; a.h = p.h; a.Wg = p.Wg; a.pos = p.pos; a.dy = p.dy; a.y = p.dx; a.dw = p.dw;
  a.B = p.B; a.T = p.T; a.D = p.D; a.K = p.K;
  a.G = (int)p.G; a.Hc = (int)(p.D / p.G); a.residual = p.residual;
  a.n_gblk = (int)(p.G / 32);
  return p.pos ? gen_bwd_by_w<true>(a, p.W, s) : gen_bwd_by_w<false>(a, p.W, s);
}

bool gen_fwd_supported(int64_t B, int64_t T, int64_t D, int64_t G, int W, int64_t K) {
  const int64_t lim = 0x7fffffff;
  if (G % 32 != 0 || D % G != 0 || (D / G) % 8 != 0 || K % kGenKS != 0 || K < kGenKS) return false;
  if (T * K * 2 >= lim || G * W * K * 2 >= lim || T * D * 2 >= lim) return false;
  // grid size at the smallest step tile (128)
  const int64_t n_tt = B * ((T + 127) / 128);
  const int64_t groups = ((n_tt + 7) / 8 + 3) / 4;
  return (int64_t)8 * groups * 4 * (G / 32) < lim;
}

template <bool POS>
hipError_t gen_by_w(const GenArgs& a, int W, hipStream_t s) {
  switch (W) {
    case 1: return gen_launch<1, POS>(a, s);
    case 2: return gen_launch<2, POS>(a, s);
    case 3: return gen_launch<3, POS>(a, s);
    case 4: return gen_launch<4, POS>(a, s);
    case 5: return gen_launch<5, POS>(a, s);
    case 6: return gen_launch<6, POS>(a, s);
    case 7: return gen_launch<7, POS>(a, s);
    default: return gen_launch<8, POS>(a, s);
  }
}

hipError_t headwise_fwd_gen(const GenProblem& p, hipStream_t s) {
  GenArgs a{};
  a.x = p.x; a.h = p.h; a.Wg = p.Wg; a.pos = p.pos; a.y = p.y;
  a.B = p.B; a.T = p.T; a.D = p.D; a.K = p.K;
  a.G = (int)p.G; a.Hc = (int)(p.D / p.G); a.residual = p.residual;
  a.n_gblk = (int)(p.G / 32);
  return p.pos ? gen_by_w<true>(a, p.W, s) : gen_by_w<false>(a, p.W, s);
}

}  // namespace dsc
