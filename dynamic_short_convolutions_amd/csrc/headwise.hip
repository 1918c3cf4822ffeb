// Head-wise entry: picks the storage-type instance set.
#include "headwise_kernels.hpp"

namespace dsc {

template <typename S>
hipError_t headwise_fwd_typed(const HeadwiseProblem&, hipStream_t);
template <typename S>
hipError_t headwise_bwd_typed(const HeadwiseProblem&, hipStream_t);

extern template hipError_t headwise_fwd_typed<bf16_t>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_fwd_typed<float>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_bwd_typed<bf16_t>(const HeadwiseProblem&, hipStream_t);
extern template hipError_t headwise_bwd_typed<float>(const HeadwiseProblem&, hipStream_t);

hipError_t headwise_fwd(const HeadwiseProblem& p, hipStream_t s) {
  return p.bf16 ? headwise_fwd_typed<bf16_t>(p, s) : headwise_fwd_typed<float>(p, s);
}

hipError_t headwise_bwd(const HeadwiseProblem& p, hipStream_t s) {
  return p.bf16 ? headwise_bwd_typed<bf16_t>(p, s) : headwise_bwd_typed<float>(p, s);
}

}  // namespace dsc
