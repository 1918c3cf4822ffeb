// Head-wise kernel instances for bf16 storage, packed sequences (positions).
#include "headwise_dispatch.hpp"

namespace dsc {

template hipError_t headwise_fwd_typed<bf16_t, true, false>(const HeadwiseProblem&, hipStream_t);
template hipError_t headwise_bwd_typed<bf16_t, true, false>(const HeadwiseProblem&, hipStream_t);

}  // namespace dsc
