// Shared device helpers for the gfx950 kernels: storage types, vector loads
// and stores, bfloat16 conversion, and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsc {

// bfloat16 is stored as its 16-bit pattern; arithmetic is always float32.
struct bf16_t {
  uint16_t bits;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// Two floats -> two bfloat16 in one dword (v_cvt_pk_bf16_f32: round to nearest-even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------------------
// 16/8-byte global accesses on native vector types. Streamed outputs are stored
// with the non-temporal hint: on MI355X that measured 3-5% faster for these
// read-then-write kernels. Loads take the hint per call site (NT): rows that
// are read once should carry it, so that they do not push out of L2 the halo
// rows a neighbouring run reads again, which must stay ordinary (every load
// non-temporal measured 5% slower, the selective choice 10% faster than none).
#ifndef DSC_LOAD_NT
#define DSC_LOAD_NT 0
#endif
#ifndef DSC_STORE_NT
#define DSC_STORE_NT 1
#endif

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename V, bool NT = (DSC_LOAD_NT != 0)>
__device__ __forceinline__ V ld_stream(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}

template <typename V, bool NT = (DSC_STORE_NT != 0)>
__device__ __forceinline__ void st_stream(void* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  else *reinterpret_cast<V*>(p) = v;
}

// ---------------------------------------------------------------------------
// 8 consecutive channels of one row ("a channel group"): 16 B of bf16 or
// 32 B of float. Loaded and stored with 16-byte vector accesses. `n4` is the
// number of valid 4-channel halves (2, or 1 for the last group of an fp32 row
// whose D is 4 mod 8).
template <typename S>
struct Group8;

template <>
struct Group8<bf16_t> {
  template <bool NT = (DSC_LOAD_NT != 0)>
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[8], int /*n4*/) {
    const u32x4_t q = ld_stream<u32x4_t, NT>(p);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[8], int /*n4*/) {
    u32x4_t q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]);
    q.w = pack_bf16x2(v[6], v[7]);
    st_stream<u32x4_t>(p, q);
  }
};

template <>
struct Group8<float> {
  template <bool NT = (DSC_LOAD_NT != 0)>
  static __device__ __forceinline__ void load(const float* p, float (&v)[8], int n4) {
    const f32x4_t a = ld_stream<f32x4_t, NT>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    if (n4 > 1) {
      const f32x4_t b = ld_stream<f32x4_t, NT>(p + 4);
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      v[4] = v[5] = v[6] = v[7] = 0.f;
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8], int n4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    if (n4 > 1) *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// ---------------------------------------------------------------------------
// N consecutive scalars (filter taps) at an address aligned to the largest
// power of two dividing N*sizeof(S) (capped at 16 B): the widest access that
// alignment allows.
template <typename S, int N>
struct Taps;

template <int N>
struct Taps<bf16_t, N> {
  static constexpr int BYTES = 2 * N;
  template <bool NT = (DSC_LOAD_NT != 0)>
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[N]) {
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        const u32x4_t q = ld_stream<u32x4_t, NT>(p + 8 * i);
        v[8 * i + 0] = bf16_lo(q.x); v[8 * i + 1] = bf16_hi(q.x);
        v[8 * i + 2] = bf16_lo(q.y); v[8 * i + 3] = bf16_hi(q.y);
        v[8 * i + 4] = bf16_lo(q.z); v[8 * i + 5] = bf16_hi(q.z);
        v[8 * i + 6] = bf16_lo(q.w); v[8 * i + 7] = bf16_hi(q.w);
      }
    } else if constexpr (BYTES % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const u32x2_t q = ld_stream<u32x2_t, NT>(p + 4 * i);
        v[4 * i + 0] = bf16_lo(q.x); v[4 * i + 1] = bf16_hi(q.x);
        v[4 * i + 2] = bf16_lo(q.y); v[4 * i + 3] = bf16_hi(q.y);
      }
    } else if constexpr (BYTES % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const uint32_t q = reinterpret_cast<const uint32_t*>(p)[i];
        v[2 * i + 0] = bf16_lo(q); v[2 * i + 1] = bf16_hi(q);
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = __uint_as_float((uint32_t)p[i].bits << 16);
    }
  }
  // Non-temporal only where a lane writes one 16-byte piece: with several, one store
  // instruction's pieces lie BYTES apart across the lanes and leave every line partly
  // written; streamed past L2 unmerged they measured 2x slower than plain stores
  // (64 bytes per lane: the taps of 8 one-channel heads).
  static constexpr bool kStoreNT = DSC_STORE_NT != 0 && BYTES <= 16;
  static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[N]) {
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        u32x4_t q;
        q.x = pack_bf16x2(v[8 * i + 0], v[8 * i + 1]);
        q.y = pack_bf16x2(v[8 * i + 2], v[8 * i + 3]);
        q.z = pack_bf16x2(v[8 * i + 4], v[8 * i + 5]);
        q.w = pack_bf16x2(v[8 * i + 6], v[8 * i + 7]);
        st_stream<u32x4_t, kStoreNT>(p + 8 * i, q);
      }
    } else if constexpr (BYTES % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        u32x2_t q;
        q.x = pack_bf16x2(v[4 * i + 0], v[4 * i + 1]);
        q.y = pack_bf16x2(v[4 * i + 2], v[4 * i + 3]);
        st_stream<u32x2_t, kStoreNT>(p + 4 * i, q);
      }
    } else if constexpr (BYTES % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) reinterpret_cast<uint32_t*>(p)[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) p[i].bits = (uint16_t)(pack_bf16x2(v[i], 0.f) & 0xffffu);
    }
  }
};

template <int N>
struct Taps<float, N> {
  static constexpr int BYTES = 4 * N;
  template <bool NT = (DSC_LOAD_NT != 0)>
  static __device__ __forceinline__ void load(const float* p, float (&v)[N]) {
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const f32x4_t q = ld_stream<f32x4_t, NT>(p + 4 * i);
        v[4 * i + 0] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
      }
    } else if constexpr (BYTES % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const f32x2_t q = ld_stream<f32x2_t, NT>(p + 2 * i);
        v[2 * i + 0] = q.x; v[2 * i + 1] = q.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = p[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[N]) {
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i)
        reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    } else if constexpr (BYTES % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) reinterpret_cast<float2*>(p)[i] = make_float2(v[2 * i], v[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) p[i] = v[i];
    }
  }
};

__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const bf16_t* p) { return __uint_as_float((uint32_t)p->bits << 16); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store1(bf16_t* p, float v) { p->bits = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu); }

}  // namespace dsc
