// Launch plan of the matrix-core low-rank kernels. The workspace query and the
// backward launch both derive their sizes from this one function.
#pragma once

#include <stddef.h>
#include <stdint.h>

// Target block counts of the forward and of the dx + dU pass (with fused dz and
// without); a build may override them for launch-size sweeps.
#ifndef DSC_LOWRANK_FWD_BLOCKS
#define DSC_LOWRANK_FWD_BLOCKS 256
#endif
#ifndef DSC_LOWRANK_BWD_BLOCKS_FUSED
#define DSC_LOWRANK_BWD_BLOCKS_FUSED 256
#endif
#ifndef DSC_LOWRANK_BWD_BLOCKS
#define DSC_LOWRANK_BWD_BLOCKS 512
#endif
// Largest rank whose dz is fused into the dx + dU pass.
#ifndef DSC_LOWRANK_FUSED_DZ_MAX_R
#define DSC_LOWRANK_FUSED_DZ_MAX_R 32
#endif

namespace dsc {

struct LowrankPlan {
  bool mfma;        // bf16, R a multiple of 8, R <= 128
  int KS, RT;       // ceil(R/32) MFMA K-steps for the filter; ceil(R/16) rank tiles
  // forward
  int fwd_QT, fwd_n_cblk, fwd_n_split;
  int64_t fwd_split_len;
  // backward, dx + dU kernel (and dz when fused: one partial per channel block)
  bool bwd_fused_dz;
  int bwd_NW;  // waves per block, 16 channels each
  int bwd_n_cblk, bwd_n_split;
  int64_t bwd_split_len;
  // backward, separate dz kernel
  int dz_MB, dz_n_rtile, dz_n_csplit;
  int64_t dz_csplit_len;
  // workspace (fp32): dU partials [B * bwd_n_split][R][D*W], then dz partials
  // [dz_parts][B*T][R] with dz_parts = bwd_n_cblk (fused) or dz_n_csplit
  int dz_parts;
  size_t dU_part_offset, dz_part_offset, workspace_bytes;
};

// Waves per block of the dx + dU kernel with fused dz: 8 (128 channels, half the dz
// partials of 4) where the LDS staging of g, z and dz of 8 waves fits in 160 KB.
constexpr int fused_dz_waves(int W) { return W <= 4 ? 8 : 4; }
// Forward: two 16-channel tiles per wave (QT = 2), each z operand feeding twice the
// MFMAs, up to 32 U operands per lane (measured faster than one tile at twice the
// occupancy for W=8, R=64).
constexpr bool fwd_pair_tiles(int W, int KS) { return 2 * W * KS <= 32; }
// Four tiles per wave (QT = 4) where the filter work is light (W * KS <= 4) and D is
// a multiple of 64: a wave then reads and writes whole 128-byte lines of each row
// (64 channels), which measured 12% faster with x streamed from HBM (92 -> 81 us at
// R=32, W=4; with x resident in the last-level cache two tiles had been faster).
constexpr bool fwd_quad_tiles(int W, int KS) { return W * KS <= 4; }
// dx + dU kernel without fused dz: two waves per channel tile, each forming g and dU
// for half of the taps, where one wave's accumulators would leave one wave per SIMD
// (R*W >= 24 with W even) and two still fit in the registers of two waves per SIMD
// (U operands W*KS plus half the dU tiles RT*W/2, in 4-register units, within 36).
constexpr int dxdU_tap_split(int W, int RT) {
  return (W % 2 == 0 && W >= 4 && RT * W >= 24 && W * ((RT + 1) / 2) + RT * W / 2 <= 36) ? 2 : 1;
}
// Blocks of 16 steps per wave of the separate dz kernels: their accumulators (MB x RT
// tiles) and staged rows stay within the registers and LDS of two waves per SIMD.
constexpr int dz_step_blocks(int RT, int W) { return RT <= 4 ? 2 : (RT * ((W + 1) & ~1) <= 40 ? 2 : 1); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }
inline int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Steps [0, T) cut into n splits of a multiple of 32 steps, about `target` blocks in total.
inline void split_steps(int64_t T, int64_t blocks_per_split, int64_t target, int* n_split, int64_t* split_len) {
  int64_t n = clamp64(ceil_div(target, blocks_per_split), 1, ceil_div(T, 32));
  int64_t len = round_up(ceil_div(T, n), 32);
  *split_len = len;
  *n_split = (int)ceil_div(T, len);
}

inline LowrankPlan make_lowrank_plan(int64_t B, int64_t T, int64_t D, int R, int W, bool bf16) {
  LowrankPlan p{};
  // per-sequence x, dy, z and the whole of U are addressed through buffer resources (< 2 GiB)
  const int64_t lim = 0x7fffffff;
  // (row offsets run up to T + 256 rows, and lanes past D add 2^31 without wrapping)
  p.mfma = bf16 && R % 8 == 0 && R >= 8 && R <= 128 && D % 8 == 0 && (T + 256) * D * 2 < lim &&
           (T + 256) * R * 2 < lim && (int64_t)R * D * W * 2 < lim;
  if (!p.mfma) return p;
  p.KS = (R + 31) / 32;
  p.RT = (R + 15) / 16;
  // Sizes below come from sweeps on MI355X at (R=32, W=4, D=2048) and (R=64, W=8, D=4096).
  // forward: 16 or 8 channels per lane (QT=4, 2) where they fit, few long blocks (the U operands
  // are loaded once per block)
  p.fwd_QT = (D % 64 == 0 && fwd_quad_tiles(W, p.KS)) ? 4 : (D % 8 == 0 && fwd_pair_tiles(W, p.KS)) ? 2 : 1;
  p.fwd_n_cblk = (int)ceil_div(D, 64 * p.fwd_QT);
  split_steps(T, (int64_t)p.fwd_n_cblk * B, DSC_LOWRANK_FWD_BLOCKS, &p.fwd_n_split, &p.fwd_split_len);
  // backward dx + dU. For R <= 32 the same pass also contracts g with U for dz: its
  // per-channel-block partials (R floats per step and channel block) cost less
  // than a second pass over x and dy. Larger ranks keep a separate dz kernel, and
  // so do sequences whose partial [T][R] (fp32, written through one buffer
  // resource) would reach 2 GiB: stores past a resource's range are dropped.
  p.bwd_fused_dz = R <= DSC_LOWRANK_FUSED_DZ_MAX_R && T * R * 4 <= lim;
  p.bwd_NW = p.bwd_fused_dz ? fused_dz_waves(W) : 4;
  p.bwd_n_cblk = (int)ceil_div(D, 16 * p.bwd_NW);
  split_steps(T, (int64_t)p.bwd_n_cblk * B, p.bwd_fused_dz ? DSC_LOWRANK_BWD_BLOCKS_FUSED : DSC_LOWRANK_BWD_BLOCKS,
              &p.bwd_n_split, &p.bwd_split_len);
  // backward dz: 4 waves x dz_MB blocks of 16 steps per block
  p.dz_MB = dz_step_blocks(p.RT, W);
  p.dz_n_rtile = (int)ceil_div(T, 64 * p.dz_MB);
  {
    int64_t n = clamp64(ceil_div(p.RT <= 2 ? 512 : 1024, (int64_t)p.dz_n_rtile * B), 1, ceil_div(D, 16));
    p.dz_csplit_len = round_up(ceil_div(D, n), 16);
    p.dz_n_csplit = (int)ceil_div(D, p.dz_csplit_len);
  }
  p.dz_parts = p.bwd_fused_dz ? p.bwd_n_cblk : p.dz_n_csplit;
  const size_t dU_bytes = (size_t)B * p.bwd_n_split * R * D * W * 4;
  const size_t dz_bytes = (size_t)p.dz_parts * B * T * R * 4;
  p.dU_part_offset = 0;
  p.dz_part_offset = (size_t)round_up((int64_t)dU_bytes, 256);
  p.workspace_bytes = p.dz_part_offset + (size_t)round_up((int64_t)dz_bytes, 256);
  // every launch of the plan within a dispatch's 32-bit work-item count; beyond it the
  // vector-ALU kernels (grid-stride loops) take the problem
  const int64_t items = (int64_t)1 << 32;
  const int64_t fwd_blocks = (int64_t)p.fwd_n_cblk * p.fwd_n_split * B;
  const int64_t bwd_blocks = (int64_t)p.bwd_n_cblk * p.bwd_n_split * B;
  const int64_t dz_blocks = (int64_t)p.dz_n_rtile * p.dz_n_csplit * B;
  const int64_t bwd_threads = p.bwd_fused_dz ? 64 * p.bwd_NW : 512;  // the unfused pass: 8 waves at most
  if (fwd_blocks * 256 >= items || bwd_blocks * bwd_threads >= items || dz_blocks * 256 >= items)
    p.mfma = false;
  return p;
}

}  // namespace dsc
