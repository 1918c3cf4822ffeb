// Matrix-core low-rank forward instances for W = 6 taps (built with MFMA results
// written straight to VGPRs; see build.py).
#include "lowrank_mfma_dispatch.hpp"

namespace dsc {

template hipError_t lowrank_mfma_fwd_w<6, false>(const LowrankProblem&, const LowrankPlan&, hipStream_t);
template hipError_t lowrank_mfma_fwd_w<6, true>(const LowrankProblem&, const LowrankPlan&, hipStream_t);

}  // namespace dsc
