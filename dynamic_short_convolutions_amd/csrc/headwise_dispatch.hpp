// Host-side dispatch of the head-wise kernels: launch shape, then the template
// instance for (storage type, taps, head layout). Instantiated once per storage
// type and per form (dense rows or packed sequences with positions, each with or
// without the rotary epilogue: headwise_{bf16,f32}{,_pos}{,_rope}.hip) so the
// eight sets compile in parallel.
#pragma once

#include "headwise_kernels.hpp"

namespace dsc {

namespace {

// Launch shape, from sweeps on MI355X (random bf16 data) at the QKV (D=6144,
// 8 channels per head) and all-linear (D=8192, 16 per head) sizes: short runs
// per thread give the most blocks in flight and the best HBM throughput despite
// the halo re-reads; loads of `unroll` steps are issued together. The DSC_*
// macros below may be set at build time for such sweeps.
constexpr int kFwdUnroll = 8;
#ifndef DSC_FWD_ROWS
#define DSC_FWD_ROWS 8
#endif
constexpr int kFwdRows = DSC_FWD_ROWS;
// Backward, one lane per head or less: runs of 12 steps, 3 per iteration (first,
// middle, last: the cache-hint policy needs W-1 <= 3 steps per iteration). Against
// runs of 8 in steps of 4 this takes 3 waves per SIMD instead of 2 for the
// instance with positions (156 registers instead of 176): packed QKV backward
// 283 -> 262 us, plain 261 -> 259 us; runs of 9 in steps of 3 were slower.
#ifndef DSC_BWD_UNROLL
#define DSC_BWD_UNROLL 3
#endif
constexpr int kBwdUnroll = DSC_BWD_UNROLL;
#ifndef DSC_BWD_ROWS
#define DSC_BWD_ROWS 12
#endif
constexpr int kBwdRows = DSC_BWD_ROWS;
// heads spanning several lanes
#ifndef DSC_BWD_UNROLL_ACROSS
#define DSC_BWD_UNROLL_ACROSS 3
#endif
#ifndef DSC_BWD_ROWS_ACROSS
#define DSC_BWD_ROWS_ACROSS 12
#endif
constexpr int kBwdUnrollAcross = DSC_BWD_UNROLL_ACROSS, kBwdRowsAcross = DSC_BWD_ROWS_ACROSS;
// with the rotary epilogue each step also holds its 8 cos and 8 sin values: the
// forward keeps fewer steps' loads in flight (4) to keep the registers (and waves
// per SIMD) of the plain kernel. The backward takes 4 like the plain one; with 2
// its cache-hint policy (which needs W-1 <= steps per iteration) was off and it
// measured 6% slower.
constexpr int kFwdUnrollRope = 4;
#ifndef DSC_BWD_UNROLL_ROPE
#define DSC_BWD_UNROLL_ROPE 4
#endif
constexpr int kBwdUnrollRope = DSC_BWD_UNROLL_ROPE;
#ifndef DSC_FWD_ROWS_ROPE
#define DSC_FWD_ROWS_ROPE 8
#endif
// the rotary backward also rotates the W-1 right-halo rows of dy again in every run:
// longer runs (16 steps) measured 4% faster there, unlike the plain kernels
#ifndef DSC_BWD_ROWS_ROPE
#define DSC_BWD_ROWS_ROPE 16
#endif
constexpr int kFwdRowsRope = DSC_FWD_ROWS_ROPE;
constexpr int kBwdRowsRope = DSC_BWD_ROWS_ROPE;

// One channel per filter (8 filters per lane): each step brings 8*W taps, so fewer
// steps' loads are in flight to keep the registers of more than one wave per SIMD.
#ifndef DSC_FWD_UNROLL_P8
#define DSC_FWD_UNROLL_P8 2
#endif
#ifndef DSC_BWD_UNROLL_P8
#define DSC_BWD_UNROLL_P8 2
#endif
#ifndef DSC_FWD_ROWS_P8
#define DSC_FWD_ROWS_P8 8
#endif
#ifndef DSC_BWD_ROWS_P8
#define DSC_BWD_ROWS_P8 12
#endif

template <typename S, bool POS, bool ROPE, int W, int MODE, int P>
hipError_t fwd_launch(const FwdArgs& a, hipStream_t s) {
  constexpr int U = ROPE ? kFwdUnrollRope : (MODE == IN_LANE && P == 8 ? DSC_FWD_UNROLL_P8 : kFwdUnroll);
  hipLaunchKernelGGL((headwise_fwd_kernel<S, W, MODE, P, U, POS, ROPE>), dim3(a.g.nblocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename S, bool POS, bool ROPE, int W, int MODE, int P>
hipError_t bwd_launch(const BwdArgs& a, hipStream_t s) {
  constexpr int U = ROPE ? kBwdUnrollRope
                         : (MODE == ACROSS ? kBwdUnrollAcross
                                           : ((MODE == IN_LANE || MODE == IN_LANE_TR) && P == 8 ? DSC_BWD_UNROLL_P8
                                                                                                : kBwdUnroll));
  hipLaunchKernelGGL((headwise_bwd_kernel<S, W, MODE, P, U, POS, ROPE>), dim3(a.g.nblocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename S, bool POS, bool ROPE, int W>
hipError_t fwd_by_layout(const FwdArgs& a, HeadLayout hl, hipStream_t s) {
  switch (hl.mode) {
    case IN_LANE:
      switch (hl.p) {
        case 8: return fwd_launch<S, POS, ROPE, W, IN_LANE, 8>(a, s);
        case 4: return fwd_launch<S, POS, ROPE, W, IN_LANE, 4>(a, s);
        case 2: return fwd_launch<S, POS, ROPE, W, IN_LANE, 2>(a, s);
        default: return fwd_launch<S, POS, ROPE, W, IN_LANE, 1>(a, s);
      }
    case ACROSS:  // the forward only needs the head index: one instance serves every P
      switch (hl.p) {
        case 2: return fwd_launch<S, POS, ROPE, W, ACROSS, 2>(a, s);
        case 4: return fwd_launch<S, POS, ROPE, W, ACROSS, 4>(a, s);
        case 8: return fwd_launch<S, POS, ROPE, W, ACROSS, 8>(a, s);
        case 16: return fwd_launch<S, POS, ROPE, W, ACROSS, 16>(a, s);
        case 32: return fwd_launch<S, POS, ROPE, W, ACROSS, 32>(a, s);
        default: return fwd_launch<S, POS, ROPE, W, ACROSS, 64>(a, s);
      }
    default:  // the rotary epilogue is built for the two layouts above (checked by the host)
      if constexpr (ROPE) return hipErrorNotSupported;
      // a group of 8 channels inside one head: the head index is all the forward needs
      // (Hc = 24 on the QKV layer: 552 -> ~151 us against per-channel tap gathers)
      else if (a.Hc % 8 == 0) return fwd_launch<S, POS, ROPE, W, ACROSS, 0>(a, s);
      else if (a.Hc > 8) return fwd_launch<S, POS, ROPE, W, GENERIC, 2>(a, s);
      else return fwd_launch<S, POS, ROPE, W, GENERIC, 1>(a, s);
  }
}

template <typename S, bool POS, bool ROPE, int W>
hipError_t bwd_by_layout(const BwdArgs& a, HeadLayout hl, hipStream_t s) {
  switch (hl.mode) {
    case IN_LANE:
      switch (hl.p) {
        case 8:
          // one channel per filter: taps through LDS where whole waves of 64 groups fit a sub-tile
          if constexpr (W == 4 && sizeof(S) == 2 && !ROPE) {
            if (a.g.cg_log2 >= 6) return bwd_launch<S, POS, ROPE, W, IN_LANE_TR, 8>(a, s);
          }
          return bwd_launch<S, POS, ROPE, W, IN_LANE, 8>(a, s);
        case 4: return bwd_launch<S, POS, ROPE, W, IN_LANE, 4>(a, s);
        case 2: return bwd_launch<S, POS, ROPE, W, IN_LANE, 2>(a, s);
        default: return bwd_launch<S, POS, ROPE, W, IN_LANE, 1>(a, s);
      }
    case ACROSS:
      switch (hl.p) {
        case 2: return bwd_launch<S, POS, ROPE, W, ACROSS, 2>(a, s);
        case 4: return bwd_launch<S, POS, ROPE, W, ACROSS, 4>(a, s);
        case 8: return bwd_launch<S, POS, ROPE, W, ACROSS, 8>(a, s);
        case 16: return bwd_launch<S, POS, ROPE, W, ACROSS, 16>(a, s);
        case 32: return bwd_launch<S, POS, ROPE, W, ACROSS, 32>(a, s);
        default: return bwd_launch<S, POS, ROPE, W, ACROSS, 64>(a, s);
      }
    default:  // dx only; dw by headwise_dw_generic_kernel (no rotary: checked by the host)
      if constexpr (ROPE) return hipErrorNotSupported;
      // whole groups of 8 channels per head: dx from the per-head taps, as in the forward
      else if (a.Hc % 8 == 0) return bwd_launch<S, POS, ROPE, W, ACROSS, 0>(a, s);
      else if (a.Hc > 8) return bwd_launch<S, POS, ROPE, W, GENERIC, 2>(a, s);
      else return bwd_launch<S, POS, ROPE, W, GENERIC, 1>(a, s);
  }
}

template <typename S, bool POS, bool ROPE>
hipError_t fwd_dispatch_w(const FwdArgs& a, int W, HeadLayout hl, hipStream_t s) {
  switch (W) {
    case 1: return fwd_by_layout<S, POS, ROPE, 1>(a, hl, s);
    case 2: return fwd_by_layout<S, POS, ROPE, 2>(a, hl, s);
    case 3: return fwd_by_layout<S, POS, ROPE, 3>(a, hl, s);
    case 4: return fwd_by_layout<S, POS, ROPE, 4>(a, hl, s);
    case 5: return fwd_by_layout<S, POS, ROPE, 5>(a, hl, s);
    case 6: return fwd_by_layout<S, POS, ROPE, 6>(a, hl, s);
    case 7: return fwd_by_layout<S, POS, ROPE, 7>(a, hl, s);
    default: return fwd_by_layout<S, POS, ROPE, 8>(a, hl, s);
  }
}

template <typename S, bool POS, bool ROPE>
hipError_t bwd_dispatch_w(const BwdArgs& a, int W, HeadLayout hl, hipStream_t s) {
  switch (W) {
    case 1: return bwd_by_layout<S, POS, ROPE, 1>(a, hl, s);
    case 2: return bwd_by_layout<S, POS, ROPE, 2>(a, hl, s);
    case 3: return bwd_by_layout<S, POS, ROPE, 3>(a, hl, s);
    case 4: return bwd_by_layout<S, POS, ROPE, 4>(a, hl, s);
    case 5: return bwd_by_layout<S, POS, ROPE, 5>(a, hl, s);
    case 6: return bwd_by_layout<S, POS, ROPE, 6>(a, hl, s);
    case 7: return bwd_by_layout<S, POS, ROPE, 7>(a, hl, s);
    default: return bwd_by_layout<S, POS, ROPE, 8>(a, hl, s);
  }
}

// Heads of 8P channels (P up to 16, not a power of two): blocks of 64P threads over
// (token, 64 heads) items, the grid capped (the kernel strides over the rest).
template <typename S, int GC>
hipError_t dw_groups_dispatch(const DwArgs& d, int W, hipStream_t s) {
  const int P = d.Hc / GC;  // P <= 16: at most 1024 threads per block
  const int64_t n = d.B * d.T * ((d.G + 63) / 64), cap = (int64_t)1 << 16;
  const dim3 grid((unsigned)(n < cap ? n : cap)), block((unsigned)(64 * P));
  const size_t lds = (size_t)64 * P * W * sizeof(float);
  switch (W) {
    case 1: hipLaunchKernelGGL((headwise_dw_groups_kernel<S, 1, GC>), grid, block, lds, s, d); break;
    case 2: hipLaunchKernelGGL((headwise_dw_groups_kernel<S, 2, GC>), grid, block, lds, s, d); break;
    case 3: hipLaunchKernelGGL((headwise_dw_groups_kernel<S, 3, GC>), grid, block, lds, s, d); break;
    case 4: hipLaunchKernelGGL((headwise_dw_groups_kernel<S, 4, GC>), grid, block, lds, s, d); break;
    case 5: hipLaunchKernelGGL((headwise_dw_groups_kernel<S, 5, GC>), grid, block, lds, s, d); break;
    case 6: hipLaunchKernelGGL((headwise_dw_groups_kernel<S, 6, GC>), grid, block, lds, s, d); break;
    case 7: hipLaunchKernelGGL((headwise_dw_groups_kernel<S, 7, GC>), grid, block, lds, s, d); break;
    default: hipLaunchKernelGGL((headwise_dw_groups_kernel<S, 8, GC>), grid, block, lds, s, d); break;
  }
  return hipGetLastError();
}

template <typename S>
hipError_t dw_generic_dispatch(const DwArgs& d, int W, hipStream_t s) {
  const int64_t n = d.B * d.T * d.G, cap = (int64_t)1 << 20;  // the kernel strides over the rest
  const dim3 grid((unsigned)((n + 255) / 256 < cap ? (n + 255) / 256 : cap));
  switch (W) {
    case 1: hipLaunchKernelGGL((headwise_dw_generic_kernel<S, 1>), grid, dim3(256), 0, s, d); break;
    case 2: hipLaunchKernelGGL((headwise_dw_generic_kernel<S, 2>), grid, dim3(256), 0, s, d); break;
    case 3: hipLaunchKernelGGL((headwise_dw_generic_kernel<S, 3>), grid, dim3(256), 0, s, d); break;
    case 4: hipLaunchKernelGGL((headwise_dw_generic_kernel<S, 4>), grid, dim3(256), 0, s, d); break;
    case 5: hipLaunchKernelGGL((headwise_dw_generic_kernel<S, 5>), grid, dim3(256), 0, s, d); break;
    case 6: hipLaunchKernelGGL((headwise_dw_generic_kernel<S, 6>), grid, dim3(256), 0, s, d); break;
    case 7: hipLaunchKernelGGL((headwise_dw_generic_kernel<S, 7>), grid, dim3(256), 0, s, d); break;
    default: hipLaunchKernelGGL((headwise_dw_generic_kernel<S, 8>), grid, dim3(256), 0, s, d); break;
  }
  return hipGetLastError();
}

}  // namespace

inline RopeArgs rope_args(const HeadwiseProblem& pr) {
  RopeArgs r{};
  if (pr.rope_cos) {
    r.cos = pr.rope_cos; r.sin = pr.rope_sin; r.n_pos = pr.rope_n_pos;
    r.rot_groups = pr.rope_d_rot / 8; r.hd = pr.rope_head_dim; r.interleaved = pr.rope_interleaved;
  }
  return r;
}

template <typename S, bool POS, bool ROPE>
hipError_t headwise_fwd_typed(const HeadwiseProblem& pr, hipStream_t s) {
  FwdArgs a;
  a.x = pr.x; a.w = pr.w; a.y = pr.y; a.pos = POS ? pr.pos : nullptr;
  a.T = pr.T; a.D = pr.D; a.G = pr.G;
  a.Hc = (int)(pr.D / pr.G);
  a.residual = pr.residual;
  a.ngroups = (int)((pr.D + 7) / 8);
  const HeadLayout hl = head_layout(a.Hc);
  const bool p8 = hl.mode == IN_LANE && hl.p == 8;
  a.g = make_tiling(pr.B, pr.T, a.ngroups,
                    pr.rows_per_thread > 0 ? pr.rows_per_thread
                                           : (ROPE ? kFwdRowsRope : (p8 ? DSC_FWD_ROWS_P8 : kFwdRows)));
  a.rope = rope_args(pr);
  return fwd_dispatch_w<S, POS, ROPE>(a, pr.W, hl, s);
}

template <typename S, bool POS, bool ROPE>
hipError_t headwise_bwd_typed(const HeadwiseProblem& pr, hipStream_t s) {
  BwdArgs a;
  a.x = pr.x; a.w = pr.w; a.pos = POS ? pr.pos : nullptr; a.dy = pr.dy; a.dx = pr.dx; a.dw = pr.dw;
  a.T = pr.T; a.D = pr.D; a.G = pr.G;
  a.Hc = (int)(pr.D / pr.G);
  a.residual = pr.residual;
  a.ngroups = (int)((pr.D + 7) / 8);
  const HeadLayout hl = head_layout(a.Hc);
  a.g = make_tiling(pr.B, pr.T, a.ngroups,
                    pr.rows_per_thread > 0 ? pr.rows_per_thread
                                           : (hl.mode == ACROSS ? kBwdRowsAcross
                                              : (ROPE ? kBwdRowsRope
                                                 : (hl.mode == IN_LANE && hl.p == 8 ? DSC_BWD_ROWS_P8 : kBwdRows))));
  a.rope = rope_args(pr);
  hipError_t e = bwd_dispatch_w<S, POS, ROPE>(a, pr.W, hl, s);
  if (e != hipSuccess || hl.mode != GENERIC) return e;
  DwArgs d{pr.x, a.pos, pr.dy, pr.dw, pr.B, pr.T, pr.D, pr.G, a.Hc};
  if (a.Hc % 8 == 0 && a.Hc <= 128) return dw_groups_dispatch<S, 8>(d, pr.W, s);
  if (a.Hc % 4 == 0 && a.Hc <= 64) return dw_groups_dispatch<S, 4>(d, pr.W, s);
  return dw_generic_dispatch<S>(d, pr.W, s);
}

}  // namespace dsc
