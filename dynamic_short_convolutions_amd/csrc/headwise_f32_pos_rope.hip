// Head-wise kernel instances with the rotary epilogue, for f32 storage, packed sequences (positions).
#include "headwise_dispatch.hpp"

namespace dsc {

template hipError_t headwise_fwd_typed<float, true, true>(const HeadwiseProblem&, hipStream_t);
template hipError_t headwise_bwd_typed<float, true, true>(const HeadwiseProblem&, hipStream_t);

}  // namespace dsc
