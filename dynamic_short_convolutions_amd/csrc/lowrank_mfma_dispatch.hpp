// Host-side launches of the matrix-core low-rank kernels for one tap count W
// (instantiated once per W, forward and backward in separate files, so they
// compile in parallel and with their own flags).
#pragma once

#include "lowrank_bwd_tr.hpp"
#include "lowrank_mfma.hpp"
#include "lowrank_plan.hpp"

namespace dsc {

namespace lowrank_detail {

inline LowrankArgs base_args(const LowrankProblem& p) {
  LowrankArgs a{};
  a.x = p.x; a.z = p.z; a.U = p.U; a.pos = p.pos; a.dy = p.dy;
  a.B = p.B; a.T = p.T; a.D = p.D; a.R = p.R; a.residual = p.residual;
  return a;
}

// blocks of 16 steps in flight per wave: deeper where the filter operands are few
template <int W, int KS, int QT, bool POS>
hipError_t fwd_launch(const LowrankArgs& a, uint32_t nblocks, hipStream_t s) {
  if constexpr (QT == 4) {
    // four tiles per wave: time in the lane (x through LDS, no lane shifts)
    hipLaunchKernelGGL((lowrank_fwd_tl_kernel<W, KS, 4, POS>), dim3(nblocks), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((lowrank_fwd_mfma_kernel<W, KS, QT, (W * KS <= 4 ? 8 : 4), POS>), dim3(nblocks), dim3(256), 0,
                       s, a);
  }
  return hipGetLastError();
}

// the channel tiles per wave must be the plan's: its block count depends on them
template <int W, int KS, bool POS>
hipError_t fwd_qt(const LowrankArgs& a, int qt, uint32_t nblocks, hipStream_t s) {
  if constexpr (fwd_quad_tiles(W, KS)) {
    if (qt == 4) return fwd_launch<W, KS, 4, POS>(a, nblocks, s);
  }
  if constexpr (fwd_pair_tiles(W, KS)) {
    if (qt == 2) return fwd_launch<W, KS, 2, POS>(a, nblocks, s);
  }
  if (qt != 1) return hipErrorInvalidValue;
  return fwd_launch<W, KS, 1, POS>(a, nblocks, s);
}

template <int W, int KS, int RT, bool POS>
hipError_t bwd_launch(const LowrankArgs& a, const LowrankPlan& pl, hipStream_t s) {
  const uint32_t nb1 = (uint32_t)((int64_t)pl.bwd_n_cblk * pl.bwd_n_split * a.B);
  if constexpr (RT <= 2) {
    if (pl.bwd_fused_dz) {
      constexpr int NW = fused_dz_waves(W);
      hipLaunchKernelGGL((lowrank_dxdU_kernel<W, KS, RT, 4, NW, true, 1, POS>), dim3(nb1), dim3(64 * NW), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (!POS && RT * W <= 40) {
    // dense sequences: x, dy, z staged in LDS, dx and dU waves paired per channel tile
    // (its dU accumulators, RT*W*4 registers, fit two waves per SIMD up to RT*W = 40)
    hipLaunchKernelGGL((lowrank_dxdU_tr_kernel<W, KS, RT>), dim3(nb1), dim3(bwd_tr::kThreads), 0, s, a);
  } else {
    // two waves per channel tile (each half of the taps) where the dU accumulators are
    // many; a shallower prefetch ring where they still take most registers
    constexpr int TS = dxdU_tap_split(W, RT);
    constexpr int PF = (TS == 2 || RT * W > 32) ? 2 : 4;
    hipLaunchKernelGGL((lowrank_dxdU_kernel<W, KS, RT, PF, 4, false, TS, POS>), dim3(nb1), dim3(256 * TS), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t nb2 = (uint32_t)((int64_t)pl.dz_n_rtile * pl.dz_n_csplit * a.B);
  constexpr int MB = dz_step_blocks(RT, W);
  if constexpr (!POS && RT * (((W + 1) & ~1) / 2) <= 16) {
    // dense sequences: x (fp32) and dy staged in LDS a line at a time, U operands per
    // 16 channels; blocks of 8 waves over row tiles of 256 steps (the plan's channel
    // splits and partials, fewer row tiles)
    LowrankArgs b = a;
    b.n_rtile = (int)ceil_div(a.T, dz_lds::kRows);
    const uint32_t nb3 = (uint32_t)((int64_t)b.n_rtile * pl.dz_n_csplit * a.B);
    hipLaunchKernelGGL((lowrank_dz_lds_kernel<W, RT>), dim3(nb3), dim3(dz_lds::kThreads), 0, s, b);
  } else {
    hipLaunchKernelGGL((lowrank_dz_kernel<W, RT, MB, POS>), dim3(nb2), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace lowrank_detail

template <int W, bool POS>
hipError_t lowrank_mfma_fwd_w(const LowrankProblem& p, const LowrankPlan& pl, hipStream_t s) {
  using namespace lowrank_detail;
  LowrankArgs a = base_args(p);
  a.out = p.y;
  a.n_cblk = pl.fwd_n_cblk;
  a.n_split = pl.fwd_n_split;
  a.split_len = pl.fwd_split_len;
  const uint32_t nb = (uint32_t)((int64_t)pl.fwd_n_cblk * pl.fwd_n_split * p.B);
  switch (pl.KS) {
    case 1: return fwd_qt<W, 1, POS>(a, pl.fwd_QT, nb, s);
    case 2: return fwd_qt<W, 2, POS>(a, pl.fwd_QT, nb, s);
    case 3: return fwd_qt<W, 3, POS>(a, pl.fwd_QT, nb, s);
    default: return fwd_qt<W, 4, POS>(a, pl.fwd_QT, nb, s);
  }
}

template <int W, bool POS>
hipError_t lowrank_mfma_bwd_w(const LowrankProblem& p, const LowrankPlan& pl, hipStream_t s) {
  using namespace lowrank_detail;
  LowrankArgs a = base_args(p);
  a.out = p.dx;
  char* ws = static_cast<char*>(p.workspace);
  a.dU_part = reinterpret_cast<float*>(ws + pl.dU_part_offset);
  a.dz_part = reinterpret_cast<float*>(ws + pl.dz_part_offset);
  a.n_cblk = pl.bwd_n_cblk;
  a.n_split = pl.bwd_n_split;
  a.split_len = pl.bwd_split_len;
  a.n_rtile = pl.dz_n_rtile;
  a.n_csplit = pl.dz_n_csplit;
  a.csplit_len = pl.dz_csplit_len;
  switch (pl.RT) {  // KS = ceil(RT/2)
    case 1: return bwd_launch<W, 1, 1, POS>(a, pl, s);
    case 2: return bwd_launch<W, 1, 2, POS>(a, pl, s);
    case 3: return bwd_launch<W, 2, 3, POS>(a, pl, s);
    case 4: return bwd_launch<W, 2, 4, POS>(a, pl, s);
    case 5: return bwd_launch<W, 3, 5, POS>(a, pl, s);
    case 6: return bwd_launch<W, 3, 6, POS>(a, pl, s);
    case 7: return bwd_launch<W, 4, 7, POS>(a, pl, s);
    default: return bwd_launch<W, 4, 8, POS>(a, pl, s);
  }
}

}  // namespace dsc
