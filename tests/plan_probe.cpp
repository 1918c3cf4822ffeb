// Host-only probe of the low-rank launch plan (csrc/lowrank_plan.hpp), built with
// g++ by tests/test_plan.py: prints the plan's fields for the sizes given on the
// command line, one `name=value` per line. No GPU code is involved.
#include <cstdio>
#include <cstdlib>

#include "lowrank_plan.hpp"

int main(int argc, char** argv) {
  if (argc != 7) {
    std::fprintf(stderr, "usage: plan_probe B T D R W bf16\n");
    return 2;
  }
  const long long B = std::atoll(argv[1]), T = std::atoll(argv[2]), D = std::atoll(argv[3]);
  const int R = std::atoi(argv[4]), W = std::atoi(argv[5]);
  const bool bf16 = std::atoi(argv[6]) != 0;
  const dsc::LowrankPlan p = dsc::make_lowrank_plan(B, T, D, R, W, bf16);
  std::printf("mfma=%d\n", (int)p.mfma);
  if (!p.mfma) return 0;
  std::printf("KS=%d\nRT=%d\n", p.KS, p.RT);
  std::printf("fwd_QT=%d\nfwd_n_cblk=%d\nfwd_n_split=%d\nfwd_split_len=%lld\n", p.fwd_QT, p.fwd_n_cblk,
              p.fwd_n_split, (long long)p.fwd_split_len);
  std::printf("bwd_fused_dz=%d\nbwd_NW=%d\nbwd_n_cblk=%d\nbwd_n_split=%d\nbwd_split_len=%lld\n",
              (int)p.bwd_fused_dz, p.bwd_NW, p.bwd_n_cblk, p.bwd_n_split, (long long)p.bwd_split_len);
  std::printf("dz_MB=%d\ndz_n_rtile=%d\ndz_n_csplit=%d\ndz_csplit_len=%lld\ndz_parts=%d\n", p.dz_MB,
              p.dz_n_rtile, p.dz_n_csplit, (long long)p.dz_csplit_len, p.dz_parts);
  std::printf("dU_part_offset=%zu\ndz_part_offset=%zu\nworkspace_bytes=%zu\n", p.dU_part_offset,
              p.dz_part_offset, p.workspace_bytes);
  return 0;
}
