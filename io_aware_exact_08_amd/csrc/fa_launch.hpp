// Host-side launchers shared by the C-ABI entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// dtype codes (same values as fa_dtype in include/flash_attn.h)
constexpr int kF16 = 0, kBF16 = 1, kF16OutF32 = 2, kBF16OutF32 = 3;

struct FwdProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;
  int N;
  int d;
  float scale;
  bool causal;
  int dtype;
  int splits = 1;         // split-KV only: key-range splits
  float* part = nullptr;  // split-KV only: partial O then partial LSE (fp32)
  int part_row_base = 0;  // split-KV only: first flattened [BH*N] row held in part
  int part_rows = 0;      // split-KV only: rows held in part (0: all BH*N)
  int item_base = 0;      // non-causal: first work item (head-major query tiles)
  int item_count = 0;     // non-causal: work items launched (0: all from item_base)
  int H = 1;              // heads per batch entry (bias addressing)
  const void* bias = nullptr;  // additive attention bias, or null
  long long bias_sb = 0, bias_sh = 0;
};

struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [BH*N] workspace: -D
  float* lse2;   // [BH*N] workspace: -LSE * log2(e)
  int BH;
  int N;
  int d;
  float scale;
  bool causal;
  int dtype;
  int H = 1;                   // heads per batch entry (bias addressing)
  const void* bias = nullptr;  // additive attention bias, or null
  long long bias_sb = 0, bias_sh = 0;
};

hipError_t launch_fwd(const FwdProblem& p, hipStream_t stream);
hipError_t launch_fwd_splitkv(const FwdProblem& p, hipStream_t stream);
int fwd_key_tile(int d);    // keys per forward tile
int fwd_query_tile(int d);  // query rows per forward workgroup
hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_pre(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdProblem& p, hipStream_t stream);

}  // namespace fa
