// Head-wise entry: picks the storage-type instance set.
#include "headwise_kernels.hpp"

namespace dsc {

template <typename S, bool POS, bool ROPE>
hipError_t headwise_fwd_typed(const HeadwiseProblem&, hipStream_t);
template <typename S, bool POS, bool ROPE>
hipError_t headwise_bwd_typed(const HeadwiseProblem&, hipStream_t);

#define DSC_EXTERN_HW(S, POS, ROPE)                                                             \
  extern template hipError_t headwise_fwd_typed<S, POS, ROPE>(const HeadwiseProblem&, hipStream_t); \
  extern template hipError_t headwise_bwd_typed<S, POS, ROPE>(const HeadwiseProblem&, hipStream_t);
DSC_EXTERN_HW(bf16_t, false, false)
DSC_EXTERN_HW(bf16_t, true, false)
DSC_EXTERN_HW(bf16_t, false, true)
DSC_EXTERN_HW(bf16_t, true, true)
DSC_EXTERN_HW(float, false, false)
DSC_EXTERN_HW(float, true, false)
DSC_EXTERN_HW(float, false, true)
DSC_EXTERN_HW(float, true, true)
#undef DSC_EXTERN_HW

template <typename S>
static hipError_t fwd_by_form(const HeadwiseProblem& p, hipStream_t s) {
  if (p.rope_cos) return p.pos ? headwise_fwd_typed<S, true, true>(p, s) : headwise_fwd_typed<S, false, true>(p, s);
  return p.pos ? headwise_fwd_typed<S, true, false>(p, s) : headwise_fwd_typed<S, false, false>(p, s);
}

template <typename S>
static hipError_t bwd_by_form(const HeadwiseProblem& p, hipStream_t s) {
  if (p.rope_cos) return p.pos ? headwise_bwd_typed<S, true, true>(p, s) : headwise_bwd_typed<S, false, true>(p, s);
  return p.pos ? headwise_bwd_typed<S, true, false>(p, s) : headwise_bwd_typed<S, false, false>(p, s);
}

hipError_t headwise_fwd(const HeadwiseProblem& p, hipStream_t s) {
  return p.bf16 ? fwd_by_form<bf16_t>(p, s) : fwd_by_form<float>(p, s);
}

hipError_t headwise_bwd(const HeadwiseProblem& p, hipStream_t s) {
  return p.bf16 ? bwd_by_form<bf16_t>(p, s) : bwd_by_form<float>(p, s);
}

}  // namespace dsc
