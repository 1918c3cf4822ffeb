// Matrix-core low-rank backward instances for W = 8 taps.
#include "lowrank_mfma_dispatch.hpp"

namespace dsc {

template hipError_t lowrank_mfma_bwd_w<8, false>(const LowrankProblem&, const LowrankPlan&, hipStream_t);

}  // namespace dsc
