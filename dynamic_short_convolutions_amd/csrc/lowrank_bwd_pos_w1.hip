// Matrix-core low-rank backward instances for W = 1 taps, packed sequences (positions).
#include "lowrank_mfma_dispatch.hpp"

namespace dsc {

template hipError_t lowrank_mfma_bwd_w<1, true>(const LowrankProblem&, const LowrankPlan&, hipStream_t);

}  // namespace dsc
