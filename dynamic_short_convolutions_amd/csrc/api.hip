// C-ABI entry points: argument validation, then dispatch to the kernel families.
// Every check happens before anything is enqueued; see include/dsc.h for the
// contract each entry point keeps.
#include <stdint.h>
#include <string.h>

#include "dsc.h"
#include "launch.hpp"

namespace {

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, int64_t elems, size_t esize) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + (uintptr_t)elems * esize};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Outputs must not overlap inputs or each other.
bool any_alias(const Span* outs, int nout, const Span* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

dsc_status_t check_common(int64_t B, int64_t T, int64_t D, int32_t W, dsc_dtype_t dt, bool* empty) {
  *empty = false;
  if (B < 0 || T < 0) return DSC_ERROR_INVALID_VALUE;
  if (B == 0 || T == 0) {
    *empty = true;
    return DSC_SUCCESS;
  }
  if (D <= 0 || W < 1 || W > 8) return DSC_ERROR_INVALID_VALUE;
  if (dt != DSC_F32 && dt != DSC_BF16) return DSC_ERROR_INVALID_VALUE;
  // keep every index computation inside int64 and the kernels' 32-bit grid
  if (B > (int64_t)1 << 31 || T > (int64_t)1 << 31 || D > (int64_t)1 << 24) return DSC_ERROR_NOT_SUPPORTED;
  if (B * T > (int64_t)1 << 34) return DSC_ERROR_NOT_SUPPORTED;
  return DSC_SUCCESS;
}

dsc_status_t check_layout(int64_t D, dsc_dtype_t dt, const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (!aligned16(ptrs[i])) return DSC_ERROR_MISALIGNED;
  if (D % (dt == DSC_BF16 ? 8 : 4) != 0) return DSC_ERROR_MISALIGNED;
  return DSC_SUCCESS;
}

bool any_null(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (!ptrs[i]) return true;
  return false;
}

size_t esize(dsc_dtype_t dt) { return dt == DSC_BF16 ? 2 : 4; }

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Checks shared by the decode entry points, after B > 0: sizes, the ring pointer
// (may be NULL only when W == 1: no ring), alignment, and the sizes the kernels'
// 32-bit grids cover (one thread per 16-byte vector of a row or of the ring).
dsc_status_t check_decode(int64_t B, int64_t D, int32_t W, dsc_dtype_t dt, const void* state) {
  if (D <= 0 || W < 1 || W > 8) return DSC_ERROR_INVALID_VALUE;
  if (dt != DSC_F32 && dt != DSC_BF16) return DSC_ERROR_INVALID_VALUE;
  if (W > 1 && !state) return DSC_ERROR_INVALID_VALUE;
  if (B > (int64_t)1 << 31 || D > (int64_t)1 << 24) return DSC_ERROR_NOT_SUPPORTED;
  if (B * D * (W > 1 ? W - 1 : 1) > (int64_t)1 << 31) return DSC_ERROR_NOT_SUPPORTED;
  return DSC_SUCCESS;
}

dsc_status_t from_hip(hipError_t e) { return e == hipSuccess ? DSC_SUCCESS : DSC_ERROR_HIP; }

}  // namespace

extern "C" {

int32_t dsc_abi_version(void) { return DSC_ABI_VERSION; }

const char* dsc_status_string(dsc_status_t s) {
  switch (s) {
    case DSC_SUCCESS: return "DSC_SUCCESS: no error";
    case DSC_ERROR_INVALID_VALUE: return "DSC_ERROR_INVALID_VALUE: a null pointer or an out-of-range size";
    case DSC_ERROR_MISALIGNED: return "DSC_ERROR_MISALIGNED: a pointer not 16-byte aligned, or D not a multiple of 8 (bf16) / 4 (fp32)";
    case DSC_ERROR_ALIASING: return "DSC_ERROR_ALIASING: an output overlaps an input or another output";
    case DSC_ERROR_NOT_SUPPORTED: return "DSC_ERROR_NOT_SUPPORTED: sizes beyond what the library handles";
    case DSC_ERROR_WORKSPACE: return "DSC_ERROR_WORKSPACE: workspace smaller than dsc_lowrank_bwd_workspace_bytes";
    case DSC_ERROR_HIP: return "DSC_ERROR_HIP: a HIP runtime call or kernel launch failed";
  }
  return "unknown dsc_status_t";
}

}  // extern "C"

namespace {

// The training entry points, with optional positions pos[B,T] (packed sequences;
// null: every row one sequence). Checks, in the documented order, then the launch.
// Rotary-embedding arguments: checked in the same order as the rest (values,
// alignment, aliasing), `ins` receives the two tables.
dsc_status_t check_rope_values(const dsc_rope_t* r, int64_t T, int64_t D, int64_t G, const int32_t* pos) {
  if (!r || !r->cos || !r->sin || r->n_pos < 1 || r->d_rot < 0 || r->d_rot > D) return DSC_ERROR_INVALID_VALUE;
  const int hd = r->head_dim;
  if (hd < 16 || hd > 512 || (hd & (hd - 1)) != 0 || r->d_rot % hd != 0) return DSC_ERROR_INVALID_VALUE;
  if (r->interleaved != 0 && r->interleaved != 1) return DSC_ERROR_INVALID_VALUE;
  if (!pos && T > r->n_pos) return DSC_ERROR_INVALID_VALUE;  // positions 0..T-1 must be in the table
  const int64_t Hc = D / G;  // filter heads: a power of two up to 512 (a layout with the rotary epilogue)
  if ((Hc & (Hc - 1)) != 0 || Hc > 512) return DSC_ERROR_NOT_SUPPORTED;
  if (r->n_pos > ((int64_t)1 << 31) / hd) return DSC_ERROR_NOT_SUPPORTED;
  return DSC_SUCCESS;
}

dsc_status_t headwise_fwd_call(const void* x, const void* w, const int32_t* pos, const dsc_rope_t* rope, void* y,
                               int64_t B, int64_t T, int64_t D, int64_t G, int32_t W, int32_t residual,
                               dsc_dtype_t dt, dsc_stream_t stream, bool need_pos) {
  bool empty;
  dsc_status_t st = check_common(B, T, D, W, dt, &empty);
  if (st != DSC_SUCCESS || empty) return st;
  if (G <= 0 || D % G != 0 || (residual != 0 && residual != 1)) return DSC_ERROR_INVALID_VALUE;
  const void* ptrs[] = {x, w, y};
  if (any_null(ptrs, 3) || (need_pos && !pos)) return DSC_ERROR_INVALID_VALUE;
  if (rope && (st = check_rope_values(rope, T, D, G, pos)) != DSC_SUCCESS) return st;
  if ((st = check_layout(D, dt, ptrs, 3)) != DSC_SUCCESS) return st;
  if (pos && !aligned4(pos)) return DSC_ERROR_MISALIGNED;
  if (rope && (!aligned16(rope->cos) || !aligned16(rope->sin))) return DSC_ERROR_MISALIGNED;
  const size_t e = esize(dt);
  Span ins[5] = {span(x, B * T * D, e), span(w, B * T * G * W, e)};
  int nin = 2;
  if (pos) ins[nin++] = span(pos, B * T, 4);
  if (rope) {
    ins[nin++] = span(rope->cos, rope->n_pos * rope->head_dim / 2, 4);
    ins[nin++] = span(rope->sin, rope->n_pos * rope->head_dim / 2, 4);
  }
  const Span outs[] = {span(y, B * T * D, e)};
  if (any_alias(outs, 1, ins, nin)) return DSC_ERROR_ALIASING;
  dsc::HeadwiseProblem p{};
  p.x = x; p.w = w; p.pos = pos; p.y = y;
  if (rope) {
    p.rope_cos = rope->cos; p.rope_sin = rope->sin; p.rope_n_pos = rope->n_pos; p.rope_d_rot = rope->d_rot;
    p.rope_head_dim = rope->head_dim; p.rope_interleaved = rope->interleaved;
  }
  p.B = B; p.T = T; p.D = D; p.G = G; p.W = W; p.residual = residual;
  p.bf16 = dt == DSC_BF16;
  return from_hip(dsc::headwise_fwd(p, static_cast<hipStream_t>(stream)));
}

dsc_status_t headwise_bwd_call(const void* x, const void* w, const int32_t* pos, const dsc_rope_t* rope,
                               const void* dy, void* dx, void* dw, int64_t B, int64_t T, int64_t D, int64_t G,
                               int32_t W, int32_t residual, dsc_dtype_t dt, dsc_stream_t stream, bool need_pos) {
  bool empty;
  dsc_status_t st = check_common(B, T, D, W, dt, &empty);
  if (st != DSC_SUCCESS || empty) return st;
  if (G <= 0 || D % G != 0 || (residual != 0 && residual != 1)) return DSC_ERROR_INVALID_VALUE;
  const void* ptrs[] = {x, w, dy, dx, dw};
  if (any_null(ptrs, 5) || (need_pos && !pos)) return DSC_ERROR_INVALID_VALUE;
  if (rope && (st = check_rope_values(rope, T, D, G, pos)) != DSC_SUCCESS) return st;
  if ((st = check_layout(D, dt, ptrs, 5)) != DSC_SUCCESS) return st;
  if (pos && !aligned4(pos)) return DSC_ERROR_MISALIGNED;
  if (rope && (!aligned16(rope->cos) || !aligned16(rope->sin))) return DSC_ERROR_MISALIGNED;
  const size_t e = esize(dt);
  Span ins[6] = {span(x, B * T * D, e), span(w, B * T * G * W, e), span(dy, B * T * D, e)};
  int nin = 3;
  if (pos) ins[nin++] = span(pos, B * T, 4);
  if (rope) {
    ins[nin++] = span(rope->cos, rope->n_pos * rope->head_dim / 2, 4);
    ins[nin++] = span(rope->sin, rope->n_pos * rope->head_dim / 2, 4);
  }
  const Span outs[] = {span(dx, B * T * D, e), span(dw, B * T * G * W, e)};
  if (any_alias(outs, 2, ins, nin)) return DSC_ERROR_ALIASING;
  dsc::HeadwiseProblem p{};
  p.x = x; p.w = w; p.pos = pos; p.dy = dy; p.dx = dx; p.dw = dw;
  if (rope) {
    p.rope_cos = rope->cos; p.rope_sin = rope->sin; p.rope_n_pos = rope->n_pos; p.rope_d_rot = rope->d_rot;
    p.rope_head_dim = rope->head_dim; p.rope_interleaved = rope->interleaved;
  }
  p.B = B; p.T = T; p.D = D; p.G = G; p.W = W; p.residual = residual;
  p.bf16 = dt == DSC_BF16;
  return from_hip(dsc::headwise_bwd(p, static_cast<hipStream_t>(stream)));
}

dsc_status_t lowrank_fwd_call(const void* x, const void* z, const void* U, const int32_t* pos, void* y, int64_t B,
                              int64_t T, int64_t D, int32_t R, int32_t W, int32_t residual, dsc_dtype_t dt,
                              dsc_stream_t stream, bool need_pos) {
  bool empty;
  dsc_status_t st = check_common(B, T, D, W, dt, &empty);
  if (st != DSC_SUCCESS || empty) return st;
  if (R < 1 || R > 128 || (residual != 0 && residual != 1)) return DSC_ERROR_INVALID_VALUE;
  const void* ptrs[] = {x, z, U, y};
  if (any_null(ptrs, 4) || (need_pos && !pos)) return DSC_ERROR_INVALID_VALUE;
  if ((st = check_layout(D, dt, ptrs, 4)) != DSC_SUCCESS) return st;
  if (pos && !aligned4(pos)) return DSC_ERROR_MISALIGNED;
  const size_t e = esize(dt);
  const Span ins[] = {span(x, B * T * D, e), span(z, B * T * R, e), span(U, (int64_t)R * D * W, e),
                      span(pos, pos ? B * T : 0, 4)};
  const Span outs[] = {span(y, B * T * D, e)};
  if (any_alias(outs, 1, ins, pos ? 4 : 3)) return DSC_ERROR_ALIASING;
  dsc::LowrankProblem p{};
  p.x = x; p.z = z; p.U = U; p.pos = pos; p.y = y;
  p.B = B; p.T = T; p.D = D; p.R = R; p.W = W; p.residual = residual;
  p.bf16 = dt == DSC_BF16;
  return from_hip(dsc::lowrank_fwd(p, static_cast<hipStream_t>(stream)));
}

// noalloc: the library's scratch array takes the place of the workspace (the
// workspace arguments are ignored; problems needing more than the array are refused).
dsc_status_t lowrank_bwd_call(const void* x, const void* z, const void* U, const int32_t* pos, const void* dy,
                              void* dx, void* dz, void* dU, void* workspace, size_t workspace_bytes, int64_t B,
                              int64_t T, int64_t D, int32_t R, int32_t W, int32_t residual, dsc_dtype_t dt,
                              dsc_stream_t stream, bool need_pos, bool noalloc = false) {
  bool empty;
  dsc_status_t st = check_common(B, T, D, W, dt, &empty);
  if (st != DSC_SUCCESS || empty) return st;
  if (R < 1 || R > 128 || (residual != 0 && residual != 1)) return DSC_ERROR_INVALID_VALUE;
  const void* ptrs[] = {x, z, U, dy, dx, dz, dU};
  if (any_null(ptrs, 7) || (need_pos && !pos)) return DSC_ERROR_INVALID_VALUE;
  if ((st = check_layout(D, dt, ptrs, 7)) != DSC_SUCCESS) return st;
  if (pos && !aligned4(pos)) return DSC_ERROR_MISALIGNED;
  const size_t need = dsc::lowrank_bwd_workspace(B, T, D, R, W, dt == DSC_BF16);
  if (noalloc) {
    if (need > dsc::kNoallocScratchBytes) return DSC_ERROR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
  } else if (need > 0) {
    if (!workspace) return DSC_ERROR_INVALID_VALUE;
    if (!aligned16(workspace)) return DSC_ERROR_MISALIGNED;
    if (workspace_bytes < need) return DSC_ERROR_WORKSPACE;
  }
  const size_t e = esize(dt);
  const Span ins[] = {span(x, B * T * D, e), span(z, B * T * R, e), span(U, (int64_t)R * D * W, e),
                      span(dy, B * T * D, e), span(pos, pos ? B * T : 0, 4)};
  Span outs[4] = {span(dx, B * T * D, e), span(dz, B * T * R, e), span(dU, (int64_t)R * D * W, e),
                  {0, 0}};
  int nout = 3;
  if (need > 0 && !noalloc)
    outs[nout++] = {reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
  if (any_alias(outs, nout, ins, pos ? 5 : 4)) return DSC_ERROR_ALIASING;
  if (noalloc && need > 0) {
    // the library's array on this device (its address is looked up once per device)
    if (dsc::lowrank_scratch(&workspace) != hipSuccess) return DSC_ERROR_HIP;
    workspace_bytes = dsc::kNoallocScratchBytes;
  }
  dsc::LowrankProblem p{};
  p.x = x; p.z = z; p.U = U; p.pos = pos; p.dy = dy; p.dx = dx; p.dz = dz; p.dU = dU;
  p.workspace = workspace; p.workspace_bytes = workspace_bytes;
  p.B = B; p.T = T; p.D = D; p.R = R; p.W = W; p.residual = residual;
  p.bf16 = dt == DSC_BF16;
  return from_hip(dsc::lowrank_bwd(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

dsc_status_t dsc_fwd(const void* x, const void* w, void* y, int64_t B, int64_t T, int64_t D, int64_t G,
                     int32_t W, int32_t residual, dsc_dtype_t dt, dsc_stream_t stream) {
  return headwise_fwd_call(x, w, nullptr, nullptr, y, B, T, D, G, W, residual, dt, stream, false);
}

dsc_status_t dsc_bwd(const void* x, const void* w, const void* dy, void* dx, void* dw, int64_t B, int64_t T,
                     int64_t D, int64_t G, int32_t W, int32_t residual, dsc_dtype_t dt, dsc_stream_t stream) {
  return headwise_bwd_call(x, w, nullptr, nullptr, dy, dx, dw, B, T, D, G, W, residual, dt, stream, false);
}

dsc_status_t dsc_lowrank_fwd(const void* x, const void* z, const void* U, void* y, int64_t B, int64_t T,
                             int64_t D, int32_t R, int32_t W, int32_t residual, dsc_dtype_t dt,
                             dsc_stream_t stream) {
  return lowrank_fwd_call(x, z, U, nullptr, y, B, T, D, R, W, residual, dt, stream, false);
}

dsc_status_t dsc_fwd_varlen(const void* x, const void* w, const int32_t* pos, void* y, int64_t B, int64_t T,
                            int64_t D, int64_t G, int32_t W, int32_t residual, dsc_dtype_t dt, dsc_stream_t stream) {
  return headwise_fwd_call(x, w, pos, nullptr, y, B, T, D, G, W, residual, dt, stream, true);
}

dsc_status_t dsc_bwd_varlen(const void* x, const void* w, const int32_t* pos, const void* dy, void* dx, void* dw,
                            int64_t B, int64_t T, int64_t D, int64_t G, int32_t W, int32_t residual, dsc_dtype_t dt,
                            dsc_stream_t stream) {
  return headwise_bwd_call(x, w, pos, nullptr, dy, dx, dw, B, T, D, G, W, residual, dt, stream, true);
}

dsc_status_t dsc_fwd_rope(const void* x, const void* w, const int32_t* pos, const dsc_rope_t* rope, void* y,
                          int64_t B, int64_t T, int64_t D, int64_t G, int32_t W, int32_t residual, dsc_dtype_t dt,
                          dsc_stream_t stream) {
  if (!rope && B > 0 && T > 0) return DSC_ERROR_INVALID_VALUE;
  return headwise_fwd_call(x, w, pos, rope, y, B, T, D, G, W, residual, dt, stream, false);
}

dsc_status_t dsc_bwd_rope(const void* x, const void* w, const int32_t* pos, const dsc_rope_t* rope, const void* dy,
                          void* dx, void* dw, int64_t B, int64_t T, int64_t D, int64_t G, int32_t W,
                          int32_t residual, dsc_dtype_t dt, dsc_stream_t stream) {
  if (!rope && B > 0 && T > 0) return DSC_ERROR_INVALID_VALUE;
  return headwise_bwd_call(x, w, pos, rope, dy, dx, dw, B, T, D, G, W, residual, dt, stream, false);
}

namespace {

dsc_status_t gen_fwd_call(const void* x, const void* h, const void* Wg, const int32_t* pos, void* y, int64_t B,
                          int64_t T, int64_t D, int64_t G, int32_t W, int64_t K, int32_t residual, dsc_dtype_t dt,
                          dsc_stream_t stream, bool need_pos) {
  bool empty;
  dsc_status_t st = check_common(B, T, D, W, dt, &empty);
  if (st != DSC_SUCCESS || empty) return st;
  if (G <= 0 || D % G != 0 || K <= 0 || (residual != 0 && residual != 1)) return DSC_ERROR_INVALID_VALUE;
  const void* ptrs[] = {x, h, Wg, y};
  if (any_null(ptrs, 4) || (need_pos && !pos)) return DSC_ERROR_INVALID_VALUE;
  if (dt != DSC_BF16 || K > ((int64_t)1 << 24) || !dsc::gen_fwd_supported(B, T, D, G, W, K))
    return DSC_ERROR_NOT_SUPPORTED;
  if ((st = check_layout(D, dt, ptrs, 4)) != DSC_SUCCESS) return st;
  if (pos && !aligned4(pos)) return DSC_ERROR_MISALIGNED;
  const size_t e = esize(dt);
  Span ins[4] = {span(x, B * T * D, e), span(h, B * T * K, e), span(Wg, G * W * K, e)};
  int nin = 3;
  if (pos) ins[nin++] = span(pos, B * T, 4);
  const Span outs[] = {span(y, B * T * D, e)};
  if (any_alias(outs, 1, ins, nin)) return DSC_ERROR_ALIASING;
  dsc::GenProblem p{};
  p.x = x; p.h = h; p.Wg = Wg; p.pos = pos; p.y = y;
  p.B = B; p.T = T; p.D = D; p.G = G; p.K = K; p.W = W; p.residual = residual;
  return from_hip(dsc::headwise_fwd_gen(p, static_cast<hipStream_t>(stream)));
}

dsc_status_t gen_bwd_call(const void* x, const void* h, const void* Wg, const int32_t* pos, const void* dy, void* dx,
                          void* dw, int64_t B, int64_t T, int64_t D, int64_t G, int32_t W, int64_t K,
                          int32_t residual, dsc_dtype_t dt, dsc_stream_t stream, bool need_pos) {
  bool empty;
  dsc_status_t st = check_common(B, T, D, W, dt, &empty);
  if (st != DSC_SUCCESS || empty) return st;
  if (G <= 0 || D % G != 0 || K <= 0 || (residual != 0 && residual != 1)) return DSC_ERROR_INVALID_VALUE;
  const void* ptrs[] = {x, h, Wg, dy, dx, dw};
  if (any_null(ptrs, 6) || (need_pos && !pos)) return DSC_ERROR_INVALID_VALUE;
  if (dt != DSC_BF16 || K > ((int64_t)1 << 24) || !dsc::gen_bwd_supported(B, T, D, G, W, K))
    return DSC_ERROR_NOT_SUPPORTED;
  if ((st = check_layout(D, dt, ptrs, 6)) != DSC_SUCCESS) return st;
  if (pos && !aligned4(pos)) return DSC_ERROR_MISALIGNED;
  const size_t e = esize(dt);
  Span ins[5] = {span(x, B * T * D, e), span(h, B * T * K, e), span(Wg, G * W * K, e), span(dy, B * T * D, e)};
  int nin = 4;
  if (pos) ins[nin++] = span(pos, B * T, 4);
  const Span outs[] = {span(dx, B * T * D, e), span(dw, B * T * G * W, e)};
  if (any_alias(outs, 2, ins, nin)) return DSC_ERROR_ALIASING;
  dsc::GenProblem p{};
  p.x = x; p.h = h; p.Wg = Wg; p.pos = pos; p.dy = dy; p.dx = dx; p.dw = dw;
  p.B = B; p.T = T; p.D = D; p.G = G; p.K = K; p.W = W; p.residual = residual;
  return from_hip(dsc::headwise_bwd_gen(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

dsc_status_t dsc_bwd_gen(const void* x, const void* h, const void* Wg, const void* dy, void* dx, void* dw, int64_t B,
                         int64_t T, int64_t D, int64_t G, int32_t W, int64_t K, int32_t residual, dsc_dtype_t dt,
                         dsc_stream_t stream) {
  return gen_bwd_call(x, h, Wg, nullptr, dy, dx, dw, B, T, D, G, W, K, residual, dt, stream, false);
}

dsc_status_t dsc_bwd_gen_varlen(const void* x, const void* h, const void* Wg, const int32_t* pos, const void* dy,
                                void* dx, void* dw, int64_t B, int64_t T, int64_t D, int64_t G, int32_t W, int64_t K,
                                int32_t residual, dsc_dtype_t dt, dsc_stream_t stream) {
  return gen_bwd_call(x, h, Wg, pos, dy, dx, dw, B, T, D, G, W, K, residual, dt, stream, true);
}

dsc_status_t dsc_fwd_gen(const void* x, const void* h, const void* Wg, void* y, int64_t B, int64_t T, int64_t D,
                         int64_t G, int32_t W, int64_t K, int32_t residual, dsc_dtype_t dt, dsc_stream_t stream) {
  return gen_fwd_call(x, h, Wg, nullptr, y, B, T, D, G, W, K, residual, dt, stream, false);
}

dsc_status_t dsc_fwd_gen_varlen(const void* x, const void* h, const void* Wg, const int32_t* pos, void* y, int64_t B,
                                int64_t T, int64_t D, int64_t G, int32_t W, int64_t K, int32_t residual,
                                dsc_dtype_t dt, dsc_stream_t stream) {
  return gen_fwd_call(x, h, Wg, pos, y, B, T, D, G, W, K, residual, dt, stream, true);
}

dsc_status_t dsc_lowrank_fwd_varlen(const void* x, const void* z, const void* U, const int32_t* pos, void* y,
                                    int64_t B, int64_t T, int64_t D, int32_t R, int32_t W, int32_t residual,
                                    dsc_dtype_t dt, dsc_stream_t stream) {
  return lowrank_fwd_call(x, z, U, pos, y, B, T, D, R, W, residual, dt, stream, true);
}

dsc_status_t dsc_lowrank_bwd_varlen(const void* x, const void* z, const void* U, const int32_t* pos, const void* dy,
                                    void* dx, void* dz, void* dU, void* workspace, size_t workspace_bytes, int64_t B,
                                    int64_t T, int64_t D, int32_t R, int32_t W, int32_t residual, dsc_dtype_t dt,
                                    dsc_stream_t stream) {
  return lowrank_bwd_call(x, z, U, pos, dy, dx, dz, dU, workspace, workspace_bytes, B, T, D, R, W, residual, dt,
                          stream, true);
}

size_t dsc_lowrank_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int32_t R, int32_t W, dsc_dtype_t dt) {
  bool empty;
  if (check_common(B, T, D, W, dt, &empty) != DSC_SUCCESS || empty) return 0;
  if (R < 1 || R > 128) return 0;
  return dsc::lowrank_bwd_workspace(B, T, D, R, W, dt == DSC_BF16);
}

dsc_status_t dsc_lowrank_bwd(const void* x, const void* z, const void* U, const void* dy, void* dx, void* dz,
                             void* dU, void* workspace, size_t workspace_bytes, int64_t B, int64_t T,
                             int64_t D, int32_t R, int32_t W, int32_t residual, dsc_dtype_t dt,
                             dsc_stream_t stream) {
  return lowrank_bwd_call(x, z, U, nullptr, dy, dx, dz, dU, workspace, workspace_bytes, B, T, D, R, W, residual, dt,
                          stream, false);
}

static_assert(DSC_NOALLOC_SCRATCH_BYTES == dsc::kNoallocScratchBytes, "scratch size in dsc.h");

dsc_status_t dsc_lowrank_bwd_noalloc(const void* x, const void* z, const void* U, const void* dy, void* dx, void* dz,
                                     void* dU, int64_t B, int64_t T, int64_t D, int32_t R, int32_t W, int32_t residual,
                                     dsc_dtype_t dt, dsc_stream_t stream) {
  return lowrank_bwd_call(x, z, U, nullptr, dy, dx, dz, dU, nullptr, 0, B, T, D, R, W, residual, dt, stream, false,
                          true);
}

dsc_status_t dsc_decode_step(const void* x, const void* w, const int32_t* pos, void* state, void* y, int64_t B,
                             int64_t D, int64_t G, int32_t W, int32_t residual, dsc_dtype_t dt,
                             dsc_stream_t stream) {
  if (B < 0) return DSC_ERROR_INVALID_VALUE;
  if (B == 0) return DSC_SUCCESS;
  dsc_status_t st = check_decode(B, D, W, dt, state);
  if (st != DSC_SUCCESS) return st;
  if (G <= 0 || D % G != 0 || (residual != 0 && residual != 1)) return DSC_ERROR_INVALID_VALUE;
  const void* ptrs[] = {x, w, y, pos};
  if (any_null(ptrs, 4)) return DSC_ERROR_INVALID_VALUE;
  const void* tensors[] = {x, w, y, W > 1 ? state : x};
  if ((st = check_layout(D, dt, tensors, 4)) != DSC_SUCCESS) return st;
  if (!aligned4(pos)) return DSC_ERROR_MISALIGNED;
  const size_t e = esize(dt);
  const Span ins[] = {span(x, B * D, e), span(w, B * G * W, e), span(pos, B, 4)};
  const Span outs[] = {span(y, B * D, e), span(state, (W - 1) * B * D, e)};
  if (any_alias(outs, W > 1 ? 2 : 1, ins, 3)) return DSC_ERROR_ALIASING;  // W == 1: no ring
  dsc::DecodeProblem p{};
  p.x = x; p.w = w; p.pos = pos; p.state = state; p.y = y;
  p.B = B; p.D = D; p.G = G; p.W = W; p.residual = residual;
  p.bf16 = dt == DSC_BF16;
  return from_hip(dsc::headwise_decode(p, static_cast<hipStream_t>(stream)));
}

dsc_status_t dsc_lowrank_decode_step(const void* x, const void* z, const void* U, const int32_t* pos, void* state,
                                     void* y, int64_t B, int64_t D, int32_t R, int32_t W, int32_t residual,
                                     dsc_dtype_t dt, dsc_stream_t stream) {
  if (B < 0) return DSC_ERROR_INVALID_VALUE;
  if (B == 0) return DSC_SUCCESS;
  dsc_status_t st = check_decode(B, D, W, dt, state);
  if (st != DSC_SUCCESS) return st;
  if (R < 1 || R > 128 || (residual != 0 && residual != 1)) return DSC_ERROR_INVALID_VALUE;
  const void* ptrs[] = {x, z, U, y, pos};
  if (any_null(ptrs, 5)) return DSC_ERROR_INVALID_VALUE;
  const void* tensors[] = {x, z, U, y, W > 1 ? state : x};
  if ((st = check_layout(D, dt, tensors, 5)) != DSC_SUCCESS) return st;
  if (!aligned4(pos)) return DSC_ERROR_MISALIGNED;
  const size_t e = esize(dt);
  const Span ins[] = {span(x, B * D, e), span(z, B * R, e), span(U, (int64_t)R * D * W, e), span(pos, B, 4)};
  const Span outs[] = {span(y, B * D, e), span(state, (W - 1) * B * D, e)};
  if (any_alias(outs, W > 1 ? 2 : 1, ins, 4)) return DSC_ERROR_ALIASING;  // W == 1: no ring
  dsc::DecodeProblem p{};
  p.x = x; p.z = z; p.U = U; p.pos = pos; p.state = state; p.y = y;
  p.B = B; p.D = D; p.R = R; p.W = W; p.residual = residual;
  p.bf16 = dt == DSC_BF16;
  return from_hip(dsc::lowrank_decode(p, static_cast<hipStream_t>(stream)));
}

dsc_status_t dsc_decode_state_from_prefill(const void* x, const int32_t* len, void* state, int64_t B, int64_t T,
                                           int64_t D, int32_t W, dsc_dtype_t dt, dsc_stream_t stream) {
  bool empty;
  dsc_status_t st = check_common(B, T, D, W, dt, &empty);
  if (st != DSC_SUCCESS || empty) return st;
  if ((st = check_decode(B, D, W, dt, state)) != DSC_SUCCESS) return st;
  if (W == 1) return DSC_SUCCESS;  // no ring
  const void* ptrs[] = {x, len};
  if (any_null(ptrs, 2)) return DSC_ERROR_INVALID_VALUE;
  const void* tensors[] = {x, state};
  if ((st = check_layout(D, dt, tensors, 2)) != DSC_SUCCESS) return st;
  if (!aligned4(len)) return DSC_ERROR_MISALIGNED;
  const size_t e = esize(dt);
  const Span ins[] = {span(x, B * T * D, e), span(len, B, 4)};
  const Span outs[] = {span(state, B * (W - 1) * D, e)};
  if (any_alias(outs, 1, ins, 2)) return DSC_ERROR_ALIASING;
  dsc::PrefillStateProblem p{};
  p.x = x; p.len = len; p.state = state;
  p.B = B; p.T = T; p.D = D; p.W = W;
  p.bf16 = dt == DSC_BF16;
  return from_hip(dsc::decode_state_from_prefill(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
