// Forward dispatch over head dimension and variant.  The kernels are in
// fa_fwd.hpp and are instantiated in slices by fa_fwd_inst.hip.
#include "fa_fwd.hpp"

namespace fa {

hipError_t launch_fwd_inst_64_0(const FwdProblem&, hipStream_t);
hipError_t launch_fwd_inst_64_1(const FwdProblem&, hipStream_t);
hipError_t launch_fwd_inst_64_2(const FwdProblem&, hipStream_t);
hipError_t launch_fwd_inst_128_0(const FwdProblem&, hipStream_t);
hipError_t launch_fwd_inst_128_1(const FwdProblem&, hipStream_t);
hipError_t launch_fwd_inst_128_2(const FwdProblem&, hipStream_t);
hipError_t launch_fwd_inst_256_0(const FwdProblem&, hipStream_t);
hipError_t launch_fwd_inst_256_1(const FwdProblem&, hipStream_t);
hipError_t launch_fwd_inst_256_2(const FwdProblem&, hipStream_t);

hipError_t launch_fwd(const FwdProblem& p, hipStream_t s) {
  const bool bias = p.bias != nullptr;
  if (p.d == 64) return bias ? launch_fwd_inst_64_1(p, s) : launch_fwd_inst_64_0(p, s);
  if (p.d == 128) return bias ? launch_fwd_inst_128_1(p, s) : launch_fwd_inst_128_0(p, s);
  if (p.d == 256) return bias ? launch_fwd_inst_256_1(p, s) : launch_fwd_inst_256_0(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_splitkv(const FwdProblem& p, hipStream_t s) {
  if (p.bias != nullptr) return hipErrorInvalidValue;
  if (p.d == 64) return launch_fwd_inst_64_2(p, s);
  if (p.d == 128) return launch_fwd_inst_128_2(p, s);
  if (p.d == 256) return launch_fwd_inst_256_2(p, s);
  return hipErrorInvalidValue;
}

int fwd_key_tile(int d) {
  return d == 64 ? FwdCfg<64>::BK : d == 128 ? FwdCfg<128>::BK : FwdCfg<256>::BK;
}
int fwd_query_tile(int d) {
  return kWaves * (d == 64 ? FwdCfg<64>::QB : d == 128 ? FwdCfg<128>::QB : FwdCfg<256>::QB) * 32;
}

}  // namespace fa
