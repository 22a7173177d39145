// C-ABI entry points: argument validation, then one enqueue on the caller's
// stream.  Declarations, argument meaning and error behaviour are documented
// in include/flash_attn.h.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/flash_attn.h"
#include "fa_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Head dimensions: 64, 128 and 256 everywhere.
bool head_dim(int d) { return d == 64 || d == 128 || d == 256; }

// The kernels address one head's rows through a buffer resource with a 32-bit
// byte range and 32-bit offsets, including the rows of a ragged last tile
// past N (up to 255 of them), whose stores the range check drops.  So every
// per-head buffer written with elements of `out_bytes` bytes must keep
// (N + 256) * d * out_bytes below 2^32; otherwise the offsets of those tail
// rows would wrap into the head's first rows.
bool head_fits_u32(int N, int d, int out_bytes) {
  return ((long long)N + 256) * d * out_bytes < (1LL << 32);
}

int check_common(int B, int H, int N, int d, float scale, int causal, int dtype, bool fwd) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (!head_dim(d)) return FA_ERR_HEADDIM;
  const long long elems = (long long)B * H * N * d;
  if (elems >= (1LL << 31)) return FA_ERR_SHAPE;
  if (dtype < FA_F16 || dtype > FA_BF16_OUT_F32) return FA_ERR_DTYPE;
  const bool o_f32 = dtype == FA_F16_OUT_F32 || dtype == FA_BF16_OUT_F32;
  // forward: O in its output type; backward: dQ, dK, dV in the input type
  if (!head_fits_u32(N, d, (fwd && o_f32) ? 4 : 2)) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  return FA_OK;
}

// ---------------------------------------------------------------------------
// Automatic split-KV plan (num_splits = 0)
// ---------------------------------------------------------------------------
// A non-causal forward is B*H*ceil(N/BQ) work items of equal length, run by
// `slots` concurrent workgroups (two per compute unit, one at d=256).  When
// the items are not a whole number of rounds, the last round leaves compute
// units idle for a whole item's time (e.g. 768 items on 512 slots take two
// rounds).  The plan compares, in units of one unsplit item's time:
//  - no split: ceil(items / slots) rounds;
//  - every item split S ways along the keys (split-KV): each split item is 1/S
//    of the work plus a fixed overhead (partial O written in fp32, pipeline
//    fill) of about four key tiles, plus the merge pass (a launch, and a read
//    of S partial rows per output row);
//  - tail split (non-causal): the whole rounds run unsplit and write O
//    directly, and only the last round's items are split S ways.
// A split plan must be 3% cheaper than no split.  Causal launches, whose
// items differ in length and are issued heaviest first, take a uniform split
// sized to shorten the heaviest item (below), at least that of
// flash_attn_fwd_splitkv_default_splits.
struct SplitPlan {
  int splits = 1;      // key-range splits of the split items
  int full_items = 0;  // items run unsplit before the split ones (tail split)
  int row_base = 0;    // first flattened [B*H*N] row of the split items
};

int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;  // MI355X
  return cus;
}

SplitPlan plan_splits(int BH, int N, int d, bool causal) {
  SplitPlan best;
  const int bq = fa::fwd_query_tile(d), bk = fa::fwd_key_tile(d);
  const int n_qt = (N + bq - 1) / bq;
  const long long items = (long long)BH * n_qt;
  const int key_tiles = (N + bk - 1) / bk;
  const long long slots = (long long)compute_units() * (d == 256 ? 1 : 2);
  if (causal) {
    // Causal items differ in length: the heaviest sees every key tile and
    // sets the launch's time when the grid is small.  Split every item into
    // the largest power of two S <= 8 that keeps items * S within one round
    // and at least 8 key tiles per range of the heaviest item; short key
    // ranges (under 2048 keys) only on grids of at most an eighth of the
    // slots, where the merge's fixed cost is repaid.  Measured (S=0 against
    // the fixed default): B1 H1 N1024 d256 37.2 -> 19.8 us, B1 H4 N1024 d128
    // bf16 26.3 -> 18.3, B1 H4 N4096 d64 35.5 -> 29.6, B1 H8 N2048 d64 25.8
    // -> 22.7; splitting B2 H12 N1024 d64 (192 items) or B2 H8 N1024 d128
    // (128 items) measured 10-30% slower.
    // Past one workgroup per compute unit the split ranges share their units,
    // which pays only over long key ranges: B2 H8 N2048 d64 (256 items)
    // measured 26.2 us unsplit and 28.2 us in two, B1 H4 N4096 d64 (128
    // items, 64 key tiles) 35.2 us in two and 29.6 us in four.
    const long long cus = compute_units();
    int S = 1;
    if (N >= 2048 || items * 8 <= slots)
      while (S < 8 && items * (2 * S) <= slots && key_tiles / (2 * S) >= 8 &&
             (items * (2 * S) <= cus || key_tiles >= 64))
        S *= 2;
    best.splits = std::max(S, flash_attn_fwd_splitkv_default_splits(1, BH, N, d, 1));
    return best;
  }
  const double tile = 1.0 / key_tiles, overhead = 4.0 * tile, merge_fixed = 4.0 * tile,
               merge_rows = 4.0 * tile;
  auto rounds = [&](long long wgs) { return (double)((wgs + slots - 1) / slots); };
  double best_cost = rounds(items);
  const double unsplit = best_cost;
  const int smax = std::min(16, key_tiles / 4);  // each split keeps at least 4 key tiles
  // The merge reads S partial rows per output row: its cost grows with S.
  // Below 64 key tiles per row the float32 partials and the merge launch cost
  // more than the model says, and a uniform split lost at B2 H12 N1024 d128
  // (192 workgroups on 512 slots); grids that fill at most an eighth of the
  // slots still gain from it (B1 H1 N1024 d256: 35.6 -> 20.3 us at S = 4).
  // Above half the slots the only gain the model sees is a partial last
  // round, which it overprices (below), so only grids of at most half the
  // slots split evenly.
  const bool short_keys = key_tiles < 64;
  const int smax_uniform = items * 2 <= slots && (!short_keys || items * 8 <= slots) ? smax : 1;
  for (int S = 2; S <= smax_uniform; ++S) {
    const double c = rounds(items * S) * (1.0 / S + overhead) + merge_fixed + merge_rows * 0.5 * S;
    if (c < best_cost && c < 0.97 * unsplit) {
      best_cost = c;
      best.splits = S;
      best.full_items = 0;
    }
  }
  const long long full = (items / slots) * slots, r = items - full;
  // A last round of up to one workgroup per compute unit runs each of them
  // without a co-resident workgroup, faster than the model's full round, so
  // the tail is split only while it fills at most a quarter of the slots.
  if (full > 0 && r > 0 && r * 4 <= slots) {
    for (int S = 2; S <= smax; ++S) {
      const double c = (double)(full / slots) + rounds(r * S) * (1.0 / S + overhead) + merge_fixed +
                       merge_rows * 0.5 * S * (double)r / (double)items;
      if (c < best_cost && c < 0.97 * unsplit) {
        best_cost = c;
        best.splits = S;
        best.full_items = (int)full;
      }
    }
  }
  best.row_base = (int)((long long)(best.full_items / n_qt) * N + (long long)(best.full_items % n_qt) * bq);
  return best;
}

// Workspace of a plan: float32 partial O and LSE of the split rows, per split.
size_t plan_workspace_bytes(const SplitPlan& pl, int BH, int N, int d) {
  if (pl.splits <= 1) return 0;
  return (size_t)pl.splits * ((size_t)BH * N - (size_t)pl.row_base) * (d + 1) * sizeof(float);
}

}  // namespace

extern "C" {

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal, dtype, true);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  fa::FwdProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = B * H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal != 0;
  p.dtype = dtype;
  return fa::launch_fwd(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int flash_attn_fwd_bias(const void* q, const void* k, const void* v, const void* bias,
                        long long bias_stride_b, long long bias_stride_h, void* o, float* lse,
                        int B, int H, int N, int d, float scale, int causal, int dtype,
                        void* stream) {
  if (!q || !k || !v || !bias || !o || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal, dtype, true);
  if (st != FA_OK) return st;
  if (N > 46340) return FA_ERR_SHAPE;  // one head's N x N bias must span < 2^32 bytes
  if (bias_stride_b < 0 || bias_stride_h < 0) return FA_ERR_SHAPE;
  const void* ptrs[] = {q, k, v, bias, o, lse};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  if (N % 8 != 0 || bias_stride_b % 8 != 0 || bias_stride_h % 8 != 0) return FA_ERR_ALIGN;
  fa::FwdProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = B * H;
  p.H = H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal != 0;
  p.dtype = dtype;
  p.bias = bias;
  p.bias_sb = bias_stride_b;
  p.bias_sh = bias_stride_h;
  return fa::launch_fwd(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t flash_attn_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits) {
  if (B < 1 || H < 1 || N < 1 || !head_dim(d)) return 0;
  if (num_splits == 0) {
    // the automatic plan, for either mask
    const size_t a = plan_workspace_bytes(plan_splits(B * H, N, d, false), B * H, N, d);
    const size_t c = plan_workspace_bytes(plan_splits(B * H, N, d, true), B * H, N, d);
    return a > c ? a : c;
  }
  if (num_splits < 1 || num_splits > 64) return 0;
  return (size_t)num_splits * B * H * N * (d + 1) * sizeof(float);
}

int flash_attn_fwd_splitkv_default_splits(int B, int H, int N, int d, int causal) {
  (void)causal;
  if (B < 1 || H < 1 || N < 1 || !head_dim(d)) return 1;
  // Splitting costs a float32 partial O per split and a merge pass, so it pays
  // only when the unsplit grid leaves compute units idle (at most one
  // workgroup per CU, 256 CUs) over long key ranges: then aim for two
  // workgroups per CU, keeping at least 32 key tiles per split (measured on
  // MI355X: B1 H4 N8192 d128 gains 1.5x at two splits, while B2 H12 N1024 d64
  // loses at any split count).
  const long long wgs = (long long)B * H * ((N + fa::fwd_query_tile(d) - 1) / fa::fwd_query_tile(d));
  const int key_tiles = (N + fa::fwd_key_tile(d) - 1) / fa::fwd_key_tile(d);
  if (wgs > 256) return 1;
  long long s = (512 + wgs - 1) / wgs;
  if (s > key_tiles / 32) s = key_tiles / 32;
  if (s > 16) s = 16;
  return s < 1 ? 1 : (int)s;
}

int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                           float scale, int causal, int dtype, int num_splits, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal, dtype, true);
  if (st != FA_OK) return st;
  if (num_splits < 0 || num_splits > 64) return FA_ERR_SPLITS;
  SplitPlan plan;
  if (num_splits == 0) {
    plan = plan_splits(B * H, N, d, causal != 0);
  } else {
    plan.splits = num_splits;
  }
  if ((long long)plan.splits * B * H * N * (d + 1) >= (1LL << 31)) return FA_ERR_SHAPE;
  if (!head_fits_u32(N, d, 4)) return FA_ERR_SHAPE;  // float32 partial O per split and head
  const size_t need = num_splits == 0 ? plan_workspace_bytes(plan, B * H, N, d)
                                      : flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  if (workspace && !aligned16(workspace)) return FA_ERR_ALIGN;
  fa::FwdProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = B * H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal != 0;
  p.dtype = dtype;
  if (plan.splits <= 1)  // (automatic plan only) nothing to split: the plain forward
    return fa::launch_fwd(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
  if (plan.full_items > 0) {
    // tail split: the whole rounds first, unsplit, writing O and LSE directly
    fa::FwdProblem pf = p;
    pf.item_count = plan.full_items;
    if (fa::launch_fwd(pf, (hipStream_t)stream) != hipSuccess) return FA_ERR_LAUNCH;
  }
  p.splits = plan.splits;
  p.part = (float*)workspace;
  p.item_base = plan.full_items;
  p.part_row_base = plan.row_base;
  p.part_rows = B * H * N - plan.row_base;
  return fa::launch_fwd_splitkv(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t flash_attn_bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  if (B < 1 || H < 1 || N < 1) return 0;
  return 2 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                   int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal, dtype, false);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < flash_attn_bwd_workspace_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  fa::BwdProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = (float*)workspace;
  p.lse2 = (float*)workspace + (size_t)B * H * N;
  p.BH = B * H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal != 0;
  p.dtype = dtype;
  return fa::launch_bwd(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int flash_attn_bwd_bias(const void* q, const void* k, const void* v, const void* bias,
                        long long bias_stride_b, long long bias_stride_h, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                        float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !bias || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal, dtype, false);
  if (st != FA_OK) return st;
  if (N > 46340 || bias_stride_b < 0 || bias_stride_h < 0) return FA_ERR_SHAPE;
  if (!workspace || workspace_bytes < flash_attn_bwd_workspace_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, bias, o, lse, dout, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  if (N % 8 != 0 || bias_stride_b % 8 != 0 || bias_stride_h % 8 != 0) return FA_ERR_ALIGN;
  fa::BwdProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = (float*)workspace;
  p.lse2 = (float*)workspace + (size_t)B * H * N;
  p.BH = B * H;
  p.H = H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal != 0;
  p.dtype = dtype;
  p.bias = bias;
  p.bias_sb = bias_stride_b;
  p.bias_sh = bias_stride_h;
  return fa::launch_bwd(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Shared checks of the three backward stages; fills p (pointers not listed
// for a stage are left NULL).
static int bwd_stage_setup(fa::BwdProblem& p, const void* workspace, size_t workspace_bytes, int B,
                           int H, int N, int d, float scale, int causal, int dtype) {
  int st = check_common(B, H, N, d, scale, causal, dtype, false);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < flash_attn_bwd_workspace_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  p = fa::BwdProblem{};
  p.delta = (float*)workspace;
  p.lse2 = (float*)workspace + (size_t)B * H * N;
  p.BH = B * H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal != 0;
  p.dtype = dtype;
  return FA_OK;
}

int flash_attn_bwd_preprocess(const void* o, const float* lse, const void* dout, void* workspace,
                              size_t workspace_bytes, int B, int H, int N, int d, int dtype,
                              void* stream) {
  if (!o || !lse || !dout) return FA_ERR_NULL;
  fa::BwdProblem p;
  int st = bwd_stage_setup(p, workspace, workspace_bytes, B, H, N, d, 1.0f, 0, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(o) || !aligned16(lse) || !aligned16(dout)) return FA_ERR_ALIGN;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  return fa::launch_bwd_pre(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                        const void* workspace, size_t workspace_bytes, void* dk, void* dv, int B,
                        int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !dout || !dk || !dv) return FA_ERR_NULL;
  fa::BwdProblem p;
  int st = bwd_stage_setup(p, workspace, workspace_bytes, B, H, N, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  const void* ptrs[] = {q, k, v, dout, dk, dv};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.dk = dk;
  p.dv = dv;
  return fa::launch_bwd_dkdv(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                      const void* workspace, size_t workspace_bytes, void* dq, int B, int H, int N,
                      int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !dout || !dq) return FA_ERR_NULL;
  fa::BwdProblem p;
  int st = bwd_stage_setup(p, workspace, workspace_bytes, B, H, N, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  const void* ptrs[] = {q, k, v, dout, dq};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.dq = dq;
  return fa::launch_bwd_dq(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free backward: the workspace of flash_attn_bwd (-D and
// -LSE*log2(e), two floats per row) in a static device array.
// ---------------------------------------------------------------------------
namespace {

static_assert(FA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
// One copy per device, alive until the process ends.  In host code `scratch`
// names a host-side handle, not a device address: kernels get the address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                           int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal, dtype, false);
  if (st != FA_OK) return st;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * N;
  if (2 * rows * sizeof(float) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return FA_ERR_LAUNCH;
  fa::BwdProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  // Every row's -D and -LSE*log2(e) are written by the preprocess before the
  // other two kernels read them, so nothing needs clearing between calls.
  p.delta = (float*)ws;
  p.lse2 = (float*)ws + rows;
  p.BH = B * H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal != 0;
  p.dtype = dtype;
  return fa::launch_bwd(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* flash_attn_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "invalid shape (B, H, N must be >= 1, tensors < 2^31 elements, (N+256)*d*(output element "
             "bytes) < 2^32 per head, causal 0/1)";
    case FA_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case FA_ERR_DTYPE: return "unknown dtype code";
    case FA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_SPLITS: return "num_splits must be between 0 (automatic) and 64";
    case FA_ERR_SCRATCH:
      return "problem too large for the allocation-free entry point's static scratch "
             "(8 * B * H * N bytes must fit FA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int flash_attn_version(void) { return 102; }

}  // extern "C"
