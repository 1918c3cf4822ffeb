// Raw buffer accesses. A buffer resource carries the size of its range, and the
// hardware returns zero for a load whose offset lies outside it, so a load that
// may fall out of range is issued without a branch by pointing its offset past
// the end (kOutOfRange). Ranges must stay below 2 GiB (offsets are 32-bit).
#pragma once

#include "common.hpp"

namespace dsc {

typedef __amdgpu_buffer_rsrc_t buf_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr uint64_t kMaxBufferBytes = 0x7fffffffu;

__device__ __forceinline__ buf_t make_buf(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < kMaxBufferBytes ? bytes : kMaxBufferBytes), 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(buf_t b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(b, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2_t buf_load8(buf_t b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(b, (int)off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_load2(buf_t b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(b, (int)off, 0, 0);
}

// Stores to an offset outside the range are dropped by the hardware. With NT the
// store is non-temporal (the output is not read again by this kernel): faster where a
// wave's rows are written at a high rate, but a 64-byte half line written slowly can
// leave L2 before the neighbouring wave's half arrives (measured: +34% bytes written).
template <bool NT>
__device__ __forceinline__ void buf_store16(buf_t b, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, b, (int)off, 0, NT ? 2 : 0);
}
template <bool NT>
__device__ __forceinline__ void buf_store8(buf_t b, uint32_t off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, b, (int)off, 0, NT ? 2 : 0);
}
// one fp32, cached (partial sums read back soon by the reduction pass)
__device__ __forceinline__ void buf_store_f32(buf_t b, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), b, (int)off, 0, 0);
}

}  // namespace dsc
