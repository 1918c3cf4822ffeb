// Internal interface between the C-ABI entry points (api.hip) and the kernel
// families. Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsc {

struct HeadwiseProblem {
  const void* x;
  const void* w;
  const int32_t* pos;  // [B, T] positions within packed sequences, or null
  const void* dy;  // backward only
  void* y;         // forward only
  void* dx;        // backward only
  void* dw;        // backward only
  int64_t B, T, D, G;
  int W, residual;
  bool bf16;
  int rows_per_thread;  // 0: default
  // rotary embedding of channels [0, rope_d_rot) after the forward (dy rotated back
  // in the backward); rope_cos null: none
  const float* rope_cos;
  const float* rope_sin;
  int64_t rope_n_pos, rope_d_rot;
  int rope_head_dim, rope_interleaved;
};

hipError_t headwise_fwd(const HeadwiseProblem& p, hipStream_t s);
hipError_t headwise_bwd(const HeadwiseProblem& p, hipStream_t s);

struct LowrankProblem {
  const void* x;
  const void* z;
  const void* U;
  const int32_t* pos;  // [B, T] positions within packed sequences, or null
  const void* dy;  // backward only
  void* y;         // forward only
  void* dx;        // backward only
  void* dz;        // backward only
  void* dU;        // backward only
  void* workspace;
  size_t workspace_bytes;
  int64_t B, T, D;
  int R, W, residual;
  bool bf16;
};

hipError_t lowrank_fwd(const LowrankProblem& p, hipStream_t s);
hipError_t lowrank_bwd(const LowrankProblem& p, hipStream_t s);
size_t lowrank_bwd_workspace(int64_t B, int64_t T, int64_t D, int R, int W, bool bf16);

// Size of the library's own scratch array, used by the allocation-free low-rank
// backward in place of a caller's workspace, and its address on the current device
// (looked up once per device).
constexpr size_t kNoallocScratchBytes = (size_t)128 << 20;
hipError_t lowrank_scratch(void** ptr);

// Head-wise forward with the filters generated from the hidden state h [B,T,K] by
// the generator weight Wg [G*W, K] in the same kernel (bf16).
struct GenProblem {
  const void* x;
  const void* h;
  const void* Wg;
  const int32_t* pos;  // [B, T] or null (packed sequences)
  void* y;             // forward
  const void* dy;      // backward
  void* dx;            // backward
  void* dw;            // backward
  int64_t B, T, D, G, K;
  int W, residual;
};

bool gen_fwd_supported(int64_t B, int64_t T, int64_t D, int64_t G, int W, int64_t K);
hipError_t headwise_fwd_gen(const GenProblem& p, hipStream_t s);
// The backward with the same filters regenerated in the kernel: dx and dw.
bool gen_bwd_supported(int64_t B, int64_t T, int64_t D, int64_t G, int W, int64_t K);
hipError_t headwise_bwd_gen(const GenProblem& p, hipStream_t s);

// One decode step: one new token per row, the previous W-1 inputs of each row in
// a ring state[B, W-1, D] (slot s mod (W-1) holds x_s), pos[b] the token's index.
struct DecodeProblem {
  const void* x;      // [B, D]
  const void* w;      // [B, G, W]   head-wise
  const void* z;      // [B, R]      low-rank
  const void* U;      // [R, D*W]    low-rank
  const int32_t* pos;  // [B]
  void* state;        // [B, W-1, D], read and written
  void* y;            // [B, D]
  int64_t B, D, G;
  int R, W, residual;
  bool bf16;
};

hipError_t headwise_decode(const DecodeProblem& p, hipStream_t s);
hipError_t lowrank_decode(const DecodeProblem& p, hipStream_t s);

// The ring after a prompt of len[b] tokens of x[B, T, D].
struct PrefillStateProblem {
  const void* x;
  const int32_t* len;
  void* state;
  int64_t B, T, D;
  int W;
  bool bf16;
};

hipError_t decode_state_from_prefill(const PrefillStateProblem& p, hipStream_t s);

}  // namespace dsc
