// Low-rank dispatch: the matrix-core kernels for bf16 with a rank that is a
// multiple of 8 (up to 128), the vector-ALU kernels for everything else.
#include <mutex>

#include "lowrank_mfma.hpp"
#include "lowrank_plan.hpp"

namespace dsc {

// ----------------------------------------------------------------------------- scratch
// The allocation-free backward keeps the reduction's fp32 partial sums here instead
// of in a caller's workspace. Each GPU the library runs on holds its own copy of the
// array until the process ends; every call on one GPU shares it, so such calls must
// not overlap. Host code never passes the array's name to a kernel: it is a host-side
// stand-in, and the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch_slots[kMaxScratchDevices];
}  // namespace

hipError_t lowrank_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch_slots[dev];
  // once per device, with that device current
  std::call_once(slot.once, [&] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
  if (slot.err != hipSuccess) return slot.err;
  *ptr = slot.ptr;
  return hipSuccess;
}

hipError_t lowrank_fwd_generic(const LowrankProblem& p, hipStream_t s);
hipError_t lowrank_bwd_generic(const LowrankProblem& p, hipStream_t s);

template <int W, bool POS>
hipError_t lowrank_mfma_fwd_w(const LowrankProblem&, const LowrankPlan&, hipStream_t);
template <int W, bool POS>
hipError_t lowrank_mfma_bwd_w(const LowrankProblem&, const LowrankPlan&, hipStream_t);

#define DSC_EXTERN_W(W)                                                                                   \
  extern template hipError_t lowrank_mfma_fwd_w<W, false>(const LowrankProblem&, const LowrankPlan&, hipStream_t); \
  extern template hipError_t lowrank_mfma_fwd_w<W, true>(const LowrankProblem&, const LowrankPlan&, hipStream_t);  \
  extern template hipError_t lowrank_mfma_bwd_w<W, false>(const LowrankProblem&, const LowrankPlan&, hipStream_t); \
  extern template hipError_t lowrank_mfma_bwd_w<W, true>(const LowrankProblem&, const LowrankPlan&, hipStream_t);
DSC_EXTERN_W(1)
DSC_EXTERN_W(2)
DSC_EXTERN_W(3)
DSC_EXTERN_W(4)
DSC_EXTERN_W(5)
DSC_EXTERN_W(6)
DSC_EXTERN_W(7)
DSC_EXTERN_W(8)
#undef DSC_EXTERN_W

size_t lowrank_bwd_workspace(int64_t B, int64_t T, int64_t D, int R, int W, bool bf16) {
  const LowrankPlan pl = make_lowrank_plan(B, T, D, R, W, bf16);
  return pl.mfma ? pl.workspace_bytes : 0;
}

template <bool POS>
static hipError_t lowrank_fwd_mfma(const LowrankProblem& p, const LowrankPlan& pl, hipStream_t s) {
  switch (p.W) {
    case 1: return lowrank_mfma_fwd_w<1, POS>(p, pl, s);
    case 2: return lowrank_mfma_fwd_w<2, POS>(p, pl, s);
    case 3: return lowrank_mfma_fwd_w<3, POS>(p, pl, s);
    case 4: return lowrank_mfma_fwd_w<4, POS>(p, pl, s);
    case 5: return lowrank_mfma_fwd_w<5, POS>(p, pl, s);
    case 6: return lowrank_mfma_fwd_w<6, POS>(p, pl, s);
    case 7: return lowrank_mfma_fwd_w<7, POS>(p, pl, s);
    default: return lowrank_mfma_fwd_w<8, POS>(p, pl, s);
  }
}

hipError_t lowrank_fwd(const LowrankProblem& p, hipStream_t s) {
  const LowrankPlan pl = make_lowrank_plan(p.B, p.T, p.D, p.R, p.W, p.bf16);
  if (!pl.mfma) return lowrank_fwd_generic(p, s);
  return p.pos ? lowrank_fwd_mfma<true>(p, pl, s) : lowrank_fwd_mfma<false>(p, pl, s);
}

// ----------------------------------------------------------------------------- reduction

// out[i] = bf16(sum_{j < parts} part[j * n + i]), summed in order j = 0, 1, ...
// Each thread takes groups of 4 elements, striding over the (capped) grid.
__device__ __forceinline__ void sum_parts_group(const float* __restrict__ part, int parts, int64_t n,
                                                bf16_t* __restrict__ out, int64_t i4) {
  if (i4 + 4 <= n && (n & 3) == 0) {
    float4 s = *reinterpret_cast<const float4*>(part + i4);
    for (int j = 1; j < parts; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)j * n + i4);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    u32x2_t q;
    q.x = pack_bf16x2(s.x, s.y);
    q.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<u32x2_t*>(out + i4) = q;
  } else {
    for (int64_t i = i4; i < n && i < i4 + 4; ++i) {
      float s = part[i];
      for (int j = 1; j < parts; ++j) s += part[(int64_t)j * n + i];
      store1(out + i, s);
    }
  }
}

__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part, int parts, int64_t n,
                                                        bf16_t* __restrict__ out) {
  for (int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i4 < n; i4 += (int64_t)gridDim.x * 256 * 4)
    sum_parts_group(part, parts, n, out, i4);
}

static hipError_t sum_parts(const float* part, int parts, int64_t n, void* out, hipStream_t s) {
  const int64_t blocks = ((n + 3) / 4 + 255) / 256;
  const int64_t cap = (int64_t)1 << 20;  // 2^28 work-items at most; the rest by striding
  hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(256), 0, s, part, parts, n,
                     static_cast<bf16_t*>(out));
  return hipGetLastError();
}

template <bool POS>
static hipError_t lowrank_bwd_mfma(const LowrankProblem& p, const LowrankPlan& pl, hipStream_t s) {
  switch (p.W) {
    case 1: return lowrank_mfma_bwd_w<1, POS>(p, pl, s);
    case 2: return lowrank_mfma_bwd_w<2, POS>(p, pl, s);
    case 3: return lowrank_mfma_bwd_w<3, POS>(p, pl, s);
    case 4: return lowrank_mfma_bwd_w<4, POS>(p, pl, s);
    case 5: return lowrank_mfma_bwd_w<5, POS>(p, pl, s);
    case 6: return lowrank_mfma_bwd_w<6, POS>(p, pl, s);
    case 7: return lowrank_mfma_bwd_w<7, POS>(p, pl, s);
    default: return lowrank_mfma_bwd_w<8, POS>(p, pl, s);
  }
}

hipError_t lowrank_bwd(const LowrankProblem& p, hipStream_t s) {
  const LowrankPlan pl = make_lowrank_plan(p.B, p.T, p.D, p.R, p.W, p.bf16);
  if (!pl.mfma) return lowrank_bwd_generic(p, s);
  hipError_t e = p.pos ? lowrank_bwd_mfma<true>(p, pl, s) : lowrank_bwd_mfma<false>(p, pl, s);
  if (e != hipSuccess) return e;
  const char* ws = static_cast<const char*>(p.workspace);
  e = sum_parts(reinterpret_cast<const float*>(ws + pl.dU_part_offset), (int)(p.B * pl.bwd_n_split),
                (int64_t)p.R * p.D * p.W, p.dU, s);
  if (e != hipSuccess) return e;
  return sum_parts(reinterpret_cast<const float*>(ws + pl.dz_part_offset), pl.dz_parts, p.B * p.T * p.R, p.dz, s);
}

}  // namespace dsc
