// Head-wise forward with the filters generated from the hidden state in the same
// kernel ("Dynamic Short Convolutions Improve Transformers", technical summary
// page, section Metodologia: the filter of step t is a learned linear map of the
// current hidden state, Parametrizacao, tied across the Hc channels of a head):
//   w[b,t,g,k] = sum_j h[b,t,j] * Wg[g*W+k, j]      (Wg: a linear layer's weight, [G*W, K])
//   y[b,t,c]   = residual*x[b,t,c] + sum_k w[b,t,c/Hc,k] * x[b,t-k,c]
// The filters live only in registers and LDS: they never reach HBM.
//
// A workgroup owns 128 steps of one sequence and 32 heads (32*W filter columns).
// It first forms its filter tile, a [128 x K] by [K x 32W] product, on the matrix
// cores (v_mfma_f32_16x16x32_bf16; A = hidden-state rows, B = generator rows, both
// K-contiguous, staged through an LDS double buffer 64 K-values at a time), then
// writes the fp32 tile to LDS and convolves the block's 32*Hc channels with it.
// Workgroups are ordered so that an XCD runs 4 step tiles against every head
// block in turn: the 4 hidden-state tiles stay in its L2 while each generator
// slice is read once per 4 step tiles.
#include "launch.hpp"
#include "lowrank_mfma.hpp"

namespace dsc {

struct GenArgs {
  const void* x;
  const void* h;
  const void* Wg;
  void* y;
  int64_t B, T, D, K;
  int G, Hc, residual;
  int n_gblk;   // head blocks of 32 heads
  int ntps;     // step tiles per sequence
  int n_tt;     // step tiles in all
  int groups;   // groups of 4 step tiles per XCD
};

constexpr int kGenM = 128;  // steps per workgroup
constexpr int kGenKS = 64;  // K values per stage

// Staged rows are 64 K-values (128 bytes, eight 16-byte chunks) with no padding;
// chunk c of row r sits at chunk position c ^ (r % 8). Eight lanes that read one
// chunk index from eight consecutive rows, or eight chunks of one row, then touch
// eight distinct 16-byte bank groups.
template <int W>
struct GenStage {
  uint16_t a[2][kGenM][kGenKS];   // hidden-state rows
  uint16_t b[2][32 * W][kGenKS];  // generator rows
};

__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ (row & 7)) * 8; }

// The filter tile, fp32: row = step, head g's W taps at g*W .. g*W+W-1; the row pitch
// stays a multiple of 16 bytes.
template <int W>
union GenShared {
  GenStage<W> g;
  float wt[kGenM][32 * W + 4];
};

template <int W>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gen_fwd_kernel(GenArgs a) {
  constexpr int NT = 32 * W;   // filter columns of the workgroup
  constexpr int NTL = NT / 16;  // MFMA column tiles
  constexpr int APER = kGenM * kGenKS / 8 / 256;  // 16-byte chunks per thread and stage: 4
  constexpr int BPER = NT * kGenKS / 8 / 256;     // W
  __shared__ __attribute__((aligned(16))) GenShared<W> sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const uint32_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const uint32_t grp = local / (4 * a.n_gblk), rr = local % (4 * a.n_gblk);
  const int gblk = (int)(rr / 4);
  const int tt = (int)((grp * 4 + rr % 4) * 8 + xcd);
  if (tt >= a.n_tt) return;  // whole workgroup, before any barrier
  const int64_t b = tt / a.ntps;
  const int t0 = (tt % a.ntps) * kGenM;
  const int64_t T = a.T, D = a.D, K = a.K;
  // per-sequence ranges below 2 GiB (checked by the host): rows past T read zero
  const buf_t hb = make_buf(static_cast<const bf16_t*>(a.h) + b * T * K, (uint64_t)(T * K * 2));
  const buf_t wb = make_buf(static_cast<const bf16_t*>(a.Wg) + (int64_t)gblk * NT * K, (uint64_t)(NT * K * 2));

  // ---------------------------------------------------------------- filter tile
  // each thread's chunks: byte offsets of stage 0 (rows past T start out of range, and
  // stay there: kOutOfRange + stage offsets is still past every resource)
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
  auto load_stage = [&](int ks, u32x4_t (&ra)[APER], u32x4_t (&rb)[BPER]) {
    const uint32_t ko = (uint32_t)(ks * kGenKS * 2);
#pragma unroll
    for (int p = 0; p < APER; ++p) ra[p] = buf_load16(hb, aoff[p] + ko);
#pragma unroll
    for (int p = 0; p < BPER; ++p) rb[p] = buf_load16(wb, boff[p] + ko);
  };
  auto store_stage = [&](int buf, const u32x4_t (&ra)[APER], const u32x4_t (&rb)[BPER]) {
#pragma unroll
    for (int p = 0; p < APER; ++p) {
      const int c = tid + 256 * p;
      *reinterpret_cast<u32x4_t*>(&sh.g.a[buf][c >> 3][swz(c >> 3, c & 7)]) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < BPER; ++p) {
      const int c = tid + 256 * p;
      *reinterpret_cast<u32x4_t*>(&sh.g.b[buf][c >> 3][swz(c >> 3, c & 7)]) = rb[p];
    }
  };

  f32x4_t acc[2][NTL];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Stage j (K values 64j .. 64j+63) is loaded into register set j % 2 two stages
  // ahead, written to LDS buffer j % 2 at the end of stage j-1, and multiplied in
  // stage j: each global load has a whole stage of products to complete in.
  const int nks = (int)(K / kGenKS);
  u32x4_t ra[2][APER], rb[2][BPER];
  load_stage(0, ra[0], rb[0]);
  if (nks > 1) load_stage(1, ra[1], rb[1]);
  store_stage(0, ra[0], rb[0]);
  __syncthreads();
  auto stage = [&](int ks, auto parc) {
    constexpr int par = decltype(parc)::value;  // ks % 2
    if (ks + 2 < nks) load_stage(ks + 2, ra[par], rb[par]);  // set par was written to LDS last stage
#pragma unroll
    for (int sub = 0; sub < kGenKS / 32; ++sub) {
      // wave: rows 32*wave .. +31 (two tiles of 16), all NT columns
      bf16x8_t av[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        av[mt] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&sh.g.a[par][32 * wave + 16 * mt + l16][swz(l16, 4 * sub + g)]));
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        const bf16x8_t bv = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&sh.g.b[par][16 * nt + l16][swz(l16, 4 * sub + g)]));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma_16x16x32(av[mt], bv, acc[mt][nt]);
      }
    }
    // stage ks+1 into the other buffer, last read in stage ks-1 (before the last barrier)
    if (ks + 1 < nks) store_stage(par ^ 1, ra[par ^ 1], rb[par ^ 1]);
    __syncthreads();
  };
  for (int ks = 0; ks < nks; ks += 2) {
    stage(ks, std::integral_constant<int, 0>{});
    if (ks + 1 < nks) stage(ks + 1, std::integral_constant<int, 1>{});
  }
  // accumulator i of tile (mt, nt): step row 32*wave + 16*mt + 4*g + i, column 16*nt + l16
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.wt[32 * wave + 16 * mt + 4 * g + i][16 * nt + l16] = acc[mt][nt][i];
  __syncthreads();

  // ---------------------------------------------------------------- convolution
  // units: (channel group of 8, slice of 16 steps); a group lies in one head (Hc % 8 == 0)
  const int ngr = 4 * a.Hc;  // 32 heads * Hc channels / 8
  const int64_t cbase = (int64_t)gblk * 32 * a.Hc;
  const bf16_t* xs = static_cast<const bf16_t*>(a.x) + b * T * D;
  bf16_t* ys = static_cast<bf16_t*>(a.y) + b * T * D;
  const float res = a.residual ? 1.f : 0.f;
  for (int u = tid; u < ngr * (kGenM / 16); u += 256) {
    const int gi = u % ngr, sl = u / ngr;
    const int head = gi * 8 / a.Hc;
    const int64_t c0 = cbase + 8 * gi;
    const int ts = t0 + 16 * sl;
    if (ts >= T) continue;
    float win[W][8];  // win[k] = x[t-k]; before step ts: the halo x[ts-1-k]
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const int r = ts - 1 - k;
      if (k < W - 1 && r >= 0) {
        Group8<bf16_t>::load(xs + (int64_t)r * D + c0, win[k], 2);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) win[k][i] = 0.f;
      }
    }
    const int te = ts + 16 < T ? ts + 16 : (int)T;
    for (int t4 = ts; t4 < te; t4 += 4) {
      float xr[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (t4 + j < te) Group8<bf16_t>::load(xs + (int64_t)(t4 + j) * D + c0, xr[j], 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t4 + j;
        if (t >= te) break;
#pragma unroll
        for (int k = W - 1; k > 0; --k)
#pragma unroll
          for (int i = 0; i < 8; ++i) win[k][i] = win[k - 1][i];
#pragma unroll
        for (int i = 0; i < 8; ++i) win[0][i] = xr[j][i];
        const float* wrow = &sh.wt[t - t0][head * W];
        float out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = res * win[0][i];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const float f = wrow[k];
#pragma unroll
          for (int i = 0; i < 8; ++i) out[i] = fmaf(f, win[k][i], out[i]);
        }
        Group8<bf16_t>::store(ys + (int64_t)t * D + c0, out, 2);
      }
    }
  }
}

namespace {

template <int W>
hipError_t gen_launch(const GenArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)8 * a.groups * 4 * a.n_gblk;
  hipLaunchKernelGGL((gen_fwd_kernel<W>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool gen_fwd_supported(int64_t B, int64_t T, int64_t D, int64_t G, int W, int64_t K) {
  const int64_t lim = 0x7fffffff;
  if (G % 32 != 0 || D % G != 0 || (D / G) % 8 != 0 || K % kGenKS != 0 || K < kGenKS) return false;
  if (T * K * 2 >= lim || G * W * K * 2 >= lim || T * D * 2 >= lim) return false;
  const int64_t n_tt = B * ((T + kGenM - 1) / kGenM);
  const int64_t groups = ((n_tt + 7) / 8 + 3) / 4;
  return (int64_t)8 * groups * 4 * (G / 32) < lim;
}

hipError_t headwise_fwd_gen(const GenProblem& p, hipStream_t s) {
  GenArgs a{};
  a.x = p.x; a.h = p.h; a.Wg = p.Wg; a.y = p.y;
  a.B = p.B; a.T = p.T; a.D = p.D; a.K = p.K;
  a.G = (int)p.G; a.Hc = (int)(p.D / p.G); a.residual = p.residual;
  a.n_gblk = (int)(p.G / 32);
  a.ntps = (int)((p.T + kGenM - 1) / kGenM);
  a.n_tt = (int)(p.B * a.ntps);
  a.groups = (int)(((a.n_tt + 7) / 8 + 3) / 4);
  switch (p.W) {
    case 1: return gen_launch<1>(a, s);
    case 2: return gen_launch<2>(a, s);
    case 3: return gen_launch<3>(a, s);
    case 4: return gen_launch<4>(a, s);
    case 5: return gen_launch<5>(a, s);
    case 6: return gen_launch<6>(a, s);
    case 7: return gen_launch<7>(a, s);
    default: return gen_launch<8>(a, s);
  }
}

}  // namespace dsc
