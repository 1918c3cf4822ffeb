// Matrix-core low-rank forward instances for W = 2 taps (built with MFMA results
// written straight to VGPRs; see build.py).
#include "lowrank_mfma_dispatch.hpp"

namespace dsc {

template hipError_t lowrank_mfma_fwd_w<2, false>(const LowrankProblem&, const LowrankPlan&, hipStream_t);
template hipError_t lowrank_mfma_fwd_w<2, true>(const LowrankProblem&, const LowrankPlan&, hipStream_t);

}  // namespace dsc
