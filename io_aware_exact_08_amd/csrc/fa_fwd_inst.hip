// One slice of the forward's kernel instantiations, chosen at compile time by
// FA_INST_D (head dimension 64, 128 or 256) and FA_INST_KIND (0: plain,
// 1: additive bias, 2: split-KV).  The build compiles this file once per
// slice, so the nine slices compile in parallel.
#include "fa_fwd.hpp"
#if FA_INST_D == 256 && FA_INST_KIND != 1
#include "fa_fwd256.hpp"
#endif

#if !defined(FA_INST_D) || !defined(FA_INST_KIND)
#error "compile with -DFA_INST_D=<64|128|256> -DFA_INST_KIND=<0|1|2>"
#endif

#define FA_INST_CAT(d, k) launch_fwd_inst_##d##_##k
#define FA_INST_NAME(d, k) FA_INST_CAT(d, k)

namespace fa {

hipError_t FA_INST_NAME(FA_INST_D, FA_INST_KIND)(const FwdProblem& p, hipStream_t s) {
#if FA_INST_D == 256 && FA_INST_KIND != 1
  // plain and split-KV d=256: the two-waves-per-SIMD kernel
  return launch_fwd256<FA_INST_KIND == 2>(p, s);
#else
  return launch_fwd_d<FA_INST_D, FA_INST_KIND == 2, FA_INST_KIND == 1>(p, s);
#endif
}

}  // namespace fa
