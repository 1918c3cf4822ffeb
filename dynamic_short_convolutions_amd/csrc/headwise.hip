// Head-wise entry: picks the storage-type instance set.
#include "headwise_kernels.hpp"

namespace dsc {

template <typename S, bool POS>
hipError_t headwise_fwd_typed(const HeadwiseProblem&, hipStream_t);
template <typename S, bool POS>
hipError_t headwise_bwd_typed(const HeadwiseProblem&, hipStream_t);

extern template hipError_t headwise_fwd_typed<bf16_t, false>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_fwd_typed<float, false>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_bwd_typed<bf16_t, false>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_bwd_typed<float, false>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_fwd_typed<bf16_t, true>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_fwd_typed<float, true>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_bwd_typed<bf16_t, true>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_bwd_typed<float, true>(const HeadwiseProblem&, hipStream_t);

hipError_t headwise_fwd(const HeadwiseProblem& p, hipStream_t s) {
  if (p.pos) return p.bf16 ? headwise_fwd_typed<bf16_t, true>(p, s) : headwise_fwd_typed<float, true>(p, s);
  return p.bf16 ? headwise_fwd_typed<bf16_t, false>(p, s) : headwise_fwd_typed<float, false>(p, s);
}

hipError_t headwise_bwd(const HeadwiseProblem& p, hipStream_t s) {
  if (p.pos) return p.bf16 ? headwise_bwd_typed<bf16_t, true>(p, s) : headwise_bwd_typed<float, true>(p, s);
  return p.bf16 ? headwise_bwd_typed<bf16_t, false>(p, s) : headwise_bwd_typed<float, false>(p, s);
}

}  // namespace dsc
