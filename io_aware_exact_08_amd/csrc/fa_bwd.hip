// Backward dispatch over head dimension.  The kernels are in fa_bwd.hpp and
// are instantiated per head dimension by fa_bwd_inst.hip.
#include "fa_bwd.hpp"

namespace fa {

#define FA_BWD_DECL(d)                                                   \
  hipError_t launch_bwd_pre_inst_##d(const BwdProblem&, hipStream_t);  \
  hipError_t launch_bwd_dkdv_inst_##d(const BwdProblem&, hipStream_t); \
  hipError_t launch_bwd_dq_inst_##d(const BwdProblem&, hipStream_t);
FA_BWD_DECL(64)
FA_BWD_DECL(128)
FA_BWD_DECL(256)
#undef FA_BWD_DECL

hipError_t launch_bwd_pre(const BwdProblem& p, hipStream_t s) {
  if (p.d == 64) return launch_bwd_pre_inst_64(p, s);
  if (p.d == 128) return launch_bwd_pre_inst_128(p, s);
  if (p.d == 256) return launch_bwd_pre_inst_256(p, s);
  return hipErrorInvalidValue;
}
hipError_t launch_bwd_dkdv(const BwdProblem& p, hipStream_t s) {
  if (p.d == 64) return launch_bwd_dkdv_inst_64(p, s);
  if (p.d == 128) return launch_bwd_dkdv_inst_128(p, s);
  if (p.d == 256) return launch_bwd_dkdv_inst_256(p, s);
  return hipErrorInvalidValue;
}
hipError_t launch_bwd_dq(const BwdProblem& p, hipStream_t s) {
  if (p.d == 64) return launch_bwd_dq_inst_64(p, s);
  if (p.d == 128) return launch_bwd_dq_inst_128(p, s);
  if (p.d == 256) return launch_bwd_dq_inst_256(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdProblem& p, hipStream_t s) {
  hipError_t e = launch_bwd_pre(p, s);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkdv(p, s);
  if (e != hipSuccess) return e;
  return launch_bwd_dq(p, s);
}

}  // namespace fa
