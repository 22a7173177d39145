// One head dimension's backward kernel instantiations, chosen at compile time
// by FA_INST_D (64, 128 or 256); the build compiles this file once per head
// dimension.
#include "fa_bwd.hpp"

#if !defined(FA_INST_D)
#error "compile with -DFA_INST_D=<64|128|256>"
#endif

#define FA_BWD_CAT(stage, d) launch_bwd_##stage##_inst_##d
#define FA_BWD_NAME(stage, d) FA_BWD_CAT(stage, d)

namespace fa {

hipError_t FA_BWD_NAME(pre, FA_INST_D)(const BwdProblem& p, hipStream_t s) {
  return dispatch_d<FA_INST_D, PreL>(p, s, p.dtype == kF16OutF32 || p.dtype == kBF16OutF32);
}
hipError_t FA_BWD_NAME(dkdv, FA_INST_D)(const BwdProblem& p, hipStream_t s) {
  return dispatch_d<FA_INST_D, DkdvL>(p, s, p.causal);
}
hipError_t FA_BWD_NAME(dq, FA_INST_D)(const BwdProblem& p, hipStream_t s) {
  return dispatch_d<FA_INST_D, DqL>(p, s, p.causal);
}

}  // namespace fa
