// Low-rank dynamic short convolution, plain vector-ALU kernels.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", technical
// summary page, section Metodologia, low-rank factorisation, and the
// fused-kernel section): the filter of channel c, tap k at step t is
//   f[b,t,c,k] = sum_r z[b,t,r] * U[r, c*W+k],
// generated in registers and used at once; it is never written to memory.
//
// These kernels serve float32 tensors and every size the matrix-core path
// does not take. Each output element is produced by one thread in a fixed
// order, so results are reproducible bit for bit. They favour simplicity:
// the bf16 configurations that matter for speed run on the MFMA kernels.
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

// Filter taps of the thread's 8 channels at one step: f[i][k] for channel 8j+i.
template <typename S, int W>
__device__ __forceinline__ void gen_filter(const S* zrow, const S* U, int64_t D, int R, int j, int n4,
                                           float (&f)[8][W]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int k = 0; k < W; ++k) f[i][k] = 0.f;
  const int64_t cols = D * W;
  const int nch = 4 * n4;
  for (int r = 0; r < R; ++r) {
    const float zr = load1(zrow + r);
    const S* urow = U + (int64_t)r * cols + (int64_t)8 * j * W;
    for (int i = 0; i < nch; ++i) {
#pragma unroll
      for (int k = 0; k < W; ++k) f[i][k] = fmaf(zr, load1(urow + i * W + k), f[i][k]);
    }
  }
}

// Tap k only: f[i] = sum_r z[r] * U[r, (8j+i)*W + k].
template <typename S>
__device__ __forceinline__ void gen_tap(const S* zrow, const S* U, int64_t D, int W, int R, int j, int n4,
                                        int k, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = 0.f;
  const int64_t cols = D * W;
  const int nch = 4 * n4;
  for (int r = 0; r < R; ++r) {
    const float zr = load1(zrow + r);
    const S* urow = U + (int64_t)r * cols + (int64_t)8 * j * W + k;
    for (int i = 0; i < nch; ++i) f[i] = fmaf(zr, load1(urow + i * W), f[i]);
  }
}

// y (one thread per step and channel group).
template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_fwd_generic_kernel(LrgArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.B * a.T * a.ngroups) return;
  const int j = (int)(idx % a.ngroups);
  const int64_t row = idx / a.ngroups, t = row % a.T;
  const int n4 = (8 * j + 4 < a.D) ? 2 : 1;
  const S* x = static_cast<const S*>(a.x);
  const int p = a.pos ? a.pos[row] : W;  // taps k > p reach into another sequence
  float f[8][W];
  gen_filter<S, W>(static_cast<const S*>(a.z) + row * a.R, static_cast<const S*>(a.U), a.D, a.R, j, n4, f);
  float out[8], xv[8];
  Group8<S>::load(x + row * a.D + 8 * j, xv, n4);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = a.residual ? xv[i] : 0.f;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    if (t - k < 0 || (k > 0 && k > p)) break;
    Group8<S>::load(x + (row - k) * a.D + 8 * j, xv, n4);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = fmaf(f[i][k], xv[i], out[i]);
  }
  Group8<S>::store(static_cast<S*>(a.out) + row * a.D + 8 * j, out, n4);
}

// dx[s] = residual*dy[s] + sum_k f(s+k)[c,k] * dy[s+k] (one thread per step and channel group).
template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_dx_generic_kernel(LrgArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.B * a.T * a.ngroups) return;
  const int j = (int)(idx % a.ngroups);
  const int64_t row = idx / a.ngroups, s = row % a.T;
  const int n4 = (8 * j + 4 < a.D) ? 2 : 1;
  const S* dy = static_cast<const S*>(a.dy);
  float out[8], dv[8];
  Group8<S>::load(dy + row * a.D + 8 * j, dv, n4);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = a.residual ? dv[i] : 0.f;
  for (int k = 0; k < W; ++k) {
    if (s + k >= a.T) break;
    if (a.pos && k > 0 && k > a.pos[row + k]) continue;  // tap k of step s+k does not exist
    float f[8];
    gen_tap<S>(static_cast<const S*>(a.z) + (row + k) * a.R, static_cast<const S*>(a.U), a.D, W, a.R, j, n4, k, f);
    Group8<S>::load(dy + (row + k) * a.D + 8 * j, dv, n4);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = fmaf(f[i], dv[i], out[i]);
  }
  Group8<S>::store(static_cast<S*>(a.out) + row * a.D + 8 * j, out, n4);
}

// dz[b,t,r] = sum_{c,k} dy[b,t,c] x[b,t-k,c] U[r,c*W+k]: one block of 256 threads per
// (token, chunk of 16 ranks); threads stride over channels, then a fixed-order tree
// in LDS finishes the sum. The sums are carried in double: the terms of these long
// contractions cancel, and an fp32 running sum loses up to its own magnitude times
// the number of terms times 2^-24, above the fp32 tolerance of a small result.
template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_dz_generic_kernel(LrgArgs a, void* dz) {
  __shared__ double red[16][256];
  const int64_t row = blockIdx.x;
  const int r0 = 16 * blockIdx.y;
  const int64_t t = row % a.T;
  const int p = a.pos ? a.pos[row] : W;
  const S* x = static_cast<const S*>(a.x);
  const S* dy = static_cast<const S*>(a.dy);
  const S* U = static_cast<const S*>(a.U);
  const int64_t cols = a.D * W;
  double acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.0;
  for (int64_t c = threadIdx.x; c < a.D; c += 256) {
    const double d = load1(dy + row * a.D + c);
    double g[W];  // exact: a product of two fp32 values
#pragma unroll
    for (int k = 0; k < W; ++k) g[k] = (t - k >= 0 && (k == 0 || k <= p)) ? d * (double)load1(x + (row - k) * a.D + c) : 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (r0 + q < a.R) {
        const S* u = U + (int64_t)(r0 + q) * cols + c * W;
#pragma unroll
        for (int k = 0; k < W; ++k) acc[q] = fma(g[k], (double)load1(u + k), acc[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) red[q][threadIdx.x] = acc[q];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w)
#pragma unroll
      for (int q = 0; q < 16; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x < 16 && r0 + (int)threadIdx.x < a.R)
    store1(static_cast<S*>(dz) + row * a.R + r0 + threadIdx.x, (float)red[threadIdx.x][0]);
}

// dU[r, c*W+k] = sum_{b,t} z[b,t,r] dy[b,t,c] x[b,t-k,c]: one thread per (column, chunk
// of 16 ranks), summing over every token in order, in double (as dz above).
template <typename S, int W>
__global__ __launch_bounds__(256) void lowrank_dU_generic_kernel(LrgArgs a, void* dU) {
  const int64_t cols = a.D * W;
  const int64_t col = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int r0 = 16 * blockIdx.y;
  if (col >= cols) return;
  const int64_t c = col / W;
  const int k = (int)(col % W);
  const S* x = static_cast<const S*>(a.x);
  const S* dy = static_cast<const S*>(a.dy);
  const S* z = static_cast<const S*>(a.z);
  double acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.0;
  for (int64_t b = 0; b < a.B; ++b) {
    for (int64_t t = k; t < a.T; ++t) {
      const int64_t row = b * a.T + t;
      if (a.pos && k > 0 && k > a.pos[row]) continue;
      const double g = (double)load1(dy + row * a.D + c) * (double)load1(x + (row - k) * a.D + c);
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (r0 + q < a.R) acc[q] = fma((double)load1(z + row * a.R + r0 + q), g, acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (r0 + q < a.R) store1(static_cast<S*>(dU) + (int64_t)(r0 + q) * cols + col, (float)acc[q]);
}

namespace {

template <typename S, int W>
hipError_t fwd_generic(const LrgArgs& a, hipStream_t s) {
  const int64_t n = a.B * a.T * a.ngroups;
  hipLaunchKernelGGL((lowrank_fwd_generic_kernel<S, W>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename S, int W>
hipError_t bwd_generic(const LrgArgs& a, void* dz, void* dU, hipStream_t s) {
  const int64_t n = a.B * a.T * a.ngroups;
  hipLaunchKernelGGL((lowrank_dx_generic_kernel<S, W>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rchunks = (unsigned)((a.R + 15) / 16);
  hipLaunchKernelGGL((lowrank_dz_generic_kernel<S, W>), dim3((unsigned)(a.B * a.T), rchunks), dim3(256), 0, s, a, dz);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cols = a.D * W;
  hipLaunchKernelGGL((lowrank_dU_generic_kernel<S, W>), dim3((unsigned)((cols + 255) / 256), rchunks), dim3(256), 0, s, a, dU);
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
