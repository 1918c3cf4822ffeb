// Head-wise kernel instances for f32 storage.
#include "headwise_dispatch.hpp"

namespace dsc {

template hipError_t headwise_fwd_typed<float, false, false>(const HeadwiseProblem&, hipStream_t);
template hipError_t headwise_bwd_typed<float, false, false>(const HeadwiseProblem&, hipStream_t);

}  // namespace dsc
