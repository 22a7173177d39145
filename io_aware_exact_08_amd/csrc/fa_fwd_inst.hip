// One slice of the forward's kernel instantiations, chosen at compile time by
// FA_INST_D (head dimension 64, 128 or 256) and FA_INST_KIND (0: plain,
// 1: additive bias, 2: split-KV).  The build compiles this file once per
// slice, so the nine slices compile in parallel.
#include "fa_fwd.hpp"
#if FA_INST_KIND != 1 && (FA_INST_D == 256 || (FA_INST_D == 128 && FA_FWD128_Q16))
#define FA_INST_Q16 1
#include "fa_fwd_q16.hpp"
#else
#define FA_INST_Q16 0
#endif

#if !defined(FA_INST_D) || !defined(FA_INST_KIND)
#error "compile with -DFA_INST_D=<64|128|256> -DFA_INST_KIND=<0|1|2>"
#endif

#define FA_INST_CAT(d, k) launch_fwd_inst_##d##_##k
#define FA_INST_NAME(d, k) FA_INST_CAT(d, k)

namespace fa {

hipError_t FA_INST_NAME(FA_INST_D, FA_INST_KIND)(const FwdProblem& p, hipStream_t s) {
#if FA_INST_Q16 && FA_INST_D == 256
  // unbiased d=256: the 16-query-wave kernel
  return launch_fwd_q16<256, FA_INST_KIND == 2>(p, s);
#elif FA_INST_Q16
  // unbiased d=128: non-causal bf16 (and every bf16 split) on the 16-query-wave
  // kernel; fp16 keeps fwd_kernel, whose lazy softmax (no row max on the
  // common path) needs more registers than the 16-query kernel has at four
  // waves per SIMD, and so does causal bf16, where fwd_kernel's mask-free
  // loop below the diagonal measured 2-5% faster
  constexpr bool SPLIT = FA_INST_KIND == 2;
  switch (p.dtype) {
    case kF16: return launch_fwd_c<128, false, false, SPLIT, false>(p, s);
    case kF16OutF32: return launch_fwd_c<128, false, true, SPLIT, false>(p, s);
    case kBF16:
      if constexpr (SPLIT) {
        return p.causal ? launch_fwd_q16_t<128, true, true, false, true>(p, s)
                        : launch_fwd_q16_t<128, true, false, false, true>(p, s);
      } else {
        return p.causal ? launch_fwd_t<128, true, true, false, false, false>(p, s)
                        : launch_fwd_q16_t<128, true, false, false, false>(p, s);
      }
    case kBF16OutF32:
      if constexpr (SPLIT) {
        return p.causal ? launch_fwd_q16_t<128, true, true, true, true>(p, s)
                        : launch_fwd_q16_t<128, true, false, true, true>(p, s);
      } else {
        return p.causal ? launch_fwd_t<128, true, true, true, false, false>(p, s)
                        : launch_fwd_q16_t<128, true, false, true, false>(p, s);
      }
    default: return hipErrorInvalidValue;
  }
#else
  return launch_fwd_d<FA_INST_D, FA_INST_KIND == 2, FA_INST_KIND == 1>(p, s);
#endif
}

}  // namespace fa
