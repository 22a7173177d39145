// Fused exact-attention forward for gfx950.
//
// Page 2 of the subject ("Kernel Fusion", "Tiling"): one kernel computes
// Q K^T, the softmax and P V for a block of query rows while K/V tiles stream
// through on-chip memory; the online softmax keeps a running row max and
// exp-sum, rescales the running sum when the max grows, and normalises once
// at the end; only O (and the row LSE the backward needs) reach HBM.
//
// Mapping onto CDNA4:
//  * A workgroup is 4 waves; each wave owns QB blocks of 32 query rows and
//    keeps their Q fragments in registers for the whole key loop.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//    lane l then holds column l%32 = one query and 16 of its keys, so the row
//    max and row sum are in-lane plus one exchange between the wave halves.
//  * K rows are fed to the MFMA with bits 2 and 3 of the row swapped, which
//    makes each lane hold 8 consecutive keys per 16-key chunk: the rounded
//    probabilities are then directly the B operand of O^T += V^T P^T.
//  * K and V tiles sit row-major in LDS, double-buffered, and are filled by
//    direct buffer->LDS loads (no staging registers): tile j+1 is in flight
//    while tile j is multiplied.  The V^T operand of O^T += V^T P^T is read
//    with the transposing ds_read_b64_tr_b16 (two per MFMA).  Both tiles use
//    16-byte-chunk XOR swizzles chosen so every operand read is free of bank
//    conflicts; the swizzle is applied by choosing each lane's source address,
//    since a direct load writes lanes to consecutive LDS slots.
//  * Global traffic uses raw buffer instructions: reads past the end of a
//    head return 0 and stores past it are dropped, so ragged tails need no
//    branches; only tiles that straddle the end or the causal diagonal run
//    the masked copy of the tile body.
//  * fp16 rescaling is lazy and needs no per-tile max: probabilities are
//    computed against the current reference and, if a row's rounded tile sum
//    exceeds 2^12 (or the tile is the first), that row alone takes an exact
//    path that raises its reference to the row max, rescales, and
//    exponentiates again.  Any common reference value gives the same
//    O = acc / l and LSE = m + log2 l exactly; the bound keeps every
//    probability far from fp16 overflow.  bf16 keeps the exact max on every
//    tile (see the threshold below).
//  * O is normalised by the sum of the probabilities as rounded for the P V
//    product (one v_dot2 per pair), so numerator and denominator carry the
//    same rounding and a dominant key's rounding error cancels.  The fp16
//    path also takes its LSE from that sum (rounding moves it by at most
//    2^-11 relative, i.e. < 5e-4 in LSE); the bf16 path keeps a second,
//    fp32 sum of the unrounded probabilities for the LSE, where a bf16 sum
//    could be off by 2^-9.
//  * An attention bias streams from HBM at two bytes per score, so its loads
//    must be in flight about two key tiles ahead.  The compiler cannot tell
//    which LDS stage a read touches while a direct load is in flight and
//    would wait for all of them before each read, so the bias kernels (d <=
//    128) issue every direct load of the key loop as inline assembly and
//    count the waits themselves; each wave stages its own bias rows in a
//    two-tile LDS ring.
//  * Non-causal launches remap workgroup ids so that all query tiles of a head
//    run on one XCD (consecutive ids are dealt round-robin over the 8 XCDs),
//    keeping that head's K/V in one L2.  Causal launches issue the heaviest
//    (last) query tiles first.
#pragma once

#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

#ifndef FA_FWD64_QB
#define FA_FWD64_QB 1
#endif
#ifndef FA_FWD64_BK
#define FA_FWD64_BK 64
#endif
#ifndef FA_FWD_STAGES
#define FA_FWD_STAGES 4
#endif
#ifndef FA_FWD_SCHED_VALU
#define FA_FWD_SCHED_VALU 12
#endif
#ifndef FA_FWD_MIN_WAVES
#define FA_FWD_MIN_WAVES 2
#endif
// Hand-counted direct loads for the unbiased d <= 128 forwards too (the
// compiler's own waits drained the next tile's loads before the first K read
// of every iteration).  Same-box A/B, bit-identical: B2 H12 N8192 d64 fp16
// -1.3 to -3.8%, bf16 -0.8%, d128 B2 H12 N4096 fp16 -7.7% and bf16 -4%.  The
// fp16 causal d=64 kernel measured +0.9 to +1.5% with them alone, and -2.5%
// (B1 H8 N16384), -9% (B2 H12 N2048, fp32 O) and +0.7% (B2 H12 N4096) with
// them and the mask-free loop below the diagonal together.
#ifndef FA_FWD_COUNTED
#define FA_FWD_COUNTED 1
#endif
// The d=256 forward runs one wave per SIMD, so the compiler's drain of the
// next tile's loads before the first LDS read of each iteration was fully
// exposed: counted loads measured -16% (B2 H8 N4096 fp16), -14% (bf16) and
// -12% (bf16 causal, fp32 O), bit-identical.
// Unbiased d=256 forwards (plain and split-KV) run fwd_q16_kernel
// (fa_fwd_q16.hpp); fwd_kernel<256> serves the biased one.  FA_FWD128_Q16
// routes the unbiased non-causal bf16 d=128 forwards and every bf16 d=128
// split there too.
#ifndef FA_FWD128_Q16
#define FA_FWD128_Q16 1
#endif
#ifndef FA_FWD256_COUNTED
#define FA_FWD256_COUNTED 1
#endif
#ifndef FA_FWD256_PREFETCH
#define FA_FWD256_PREFETCH 0
#endif

template <int D>
struct FwdCfg;
template <>
struct FwdCfg<64> {
  static constexpr int QB = FA_FWD64_QB;  // 32-row query blocks per wave
  static constexpr int BK = FA_FWD64_BK;  // keys per tile
  static constexpr int STAGES = FA_FWD_STAGES;        // K/V tiles resident in LDS
  static constexpr bool Q_LDS = false;                // Q^T operand from LDS (else registers)
  static constexpr bool PREFETCH = true;              // next tile's scores during this softmax
  static constexpr bool PIN = false;                  // operand reads pinned FA_FWD_PIN_LA ahead
  static constexpr int MIN_WAVES = FA_FWD_MIN_WAVES;  // waves per SIMD the registers allow
};
template <>
struct FwdCfg<128> {
  static constexpr int QB = 1;
  static constexpr int BK = 32;
  static constexpr int STAGES = FA_FWD_STAGES;
  static constexpr bool Q_LDS = false;
  static constexpr bool PREFETCH = true;
  // Pinned reads remove the 15-20 VGPR spills of the d=128 instantiations:
  // -3.8% at B2 H16 N4096 bf16 causal (at d=64 it measured +2.2% causal, -0.8%
  // non-causal, so d=64 keeps the free schedule).
  static constexpr bool PIN = true;
  static constexpr int MIN_WAVES = FA_FWD_MIN_WAVES;
};
// d=256: the O^T accumulators alone take 128 registers per lane, so the Q^T
// operand is read from LDS instead of being held in 64 more (with it in
// registers the accumulators no longer fit in VGPRs, and every online-softmax
// rescale of AGPR-resident accumulators spills).  Q (64 KB) plus three 32-key
// stages of K and V (96 KB) fill the CU's 160 KB of LDS: one workgroup per CU,
// one wave per SIMD.  MFMA work per key tile is 4x that of d=64 while the
// softmax work is the same, so that single wave keeps the matrix core busy.
template <>
struct FwdCfg<256> {
  static constexpr int QB = 1;
  static constexpr int BK = 32;
  static constexpr int STAGES = 3;
  static constexpr bool Q_LDS = true;
  static constexpr bool PREFETCH = FA_FWD256_PREFETCH;
  static constexpr bool PIN = false;  // (the LDS-resident Q path pins its own reads)
  static constexpr int MIN_WAVES = 1;
};

constexpr int kWaves = 4;
// wave priority of the fp16 score/exponential phase (see softmax_pv)
#ifndef FA_FWD_PRIO_SCORES
#define FA_FWD_PRIO_SCORES 1
#endif
constexpr int kPrioScores = FA_FWD_PRIO_SCORES;
constexpr int kThreads = kWaves * 64;

// Lazy-rescale threshold (log2 units).  bf16 keeps the exact running max
// (threshold 0): the dominant probability is then exactly 1 and is not
// rounded, which matters with 8-bit mantissas when one key dominates a row.
template <bool BF16>
constexpr float rescale_threshold() { return BF16 ? 0.0f : 8.0f; }
// fp16 fast path: largest row sum of rounded probabilities per tile that
// keeps the current reference.
constexpr float kLazyBound = 4096.0f;
// fp16 reference of a row that has seen no visible key: finite (no NaN from
// -inf - -inf) and far below any score.
constexpr float kNoReference = -1.0e30f;

#ifndef FA_QLDS_LOOKAHEAD
#define FA_QLDS_LOOKAHEAD 4
#endif
#ifndef FA_FWD_PIN_LA
#define FA_FWD_PIN_LA 4
#endif
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int N;
  int BH;
  int n_qtiles;
  float c;  // scale * log2(e)
  // split-KV: the key tiles of each query tile are cut into `splits` ranges;
  // each workgroup writes its range's O (fp32, normalised by its own sum) and
  // LSE to part_o [splits][part_rows][D] and part_lse [splits][part_rows],
  // partial row r holding row part_row_base + r of the flattened [BH*N].
  int splits;
  float* part_o;
  float* part_lse;
  int part_row_base, part_rows;
  // non-causal launches cover work items item_base .. item_base + grid/splits
  // - 1, item i being query tile i % n_qtiles of head i / n_qtiles
  int item_base;
  // additive attention bias (input type, [N][N] rows per (b, h) at element
  // offset b*bias_sb + h*bias_sh; 0 strides broadcast)
  const uint16_t* bias;
  long long bias_sb, bias_sh;
  int H;
};

template <int D, bool BF16, bool CAUSAL, bool OUT_F32, bool SPLITKV, bool BIAS>
__global__ __launch_bounds__(kThreads, FwdCfg<D>::MIN_WAVES) void fwd_kernel(FwdArgs a) {
  constexpr int QB = FwdCfg<D>::QB;
  constexpr int BK = FwdCfg<D>::BK;
  constexpr int BQ = kWaves * QB * 32;
  constexpr int DC = D / 16;   // 16-wide d chunks (contraction of S^T)
  constexpr int DT = D / 32;   // 32-row d tiles of O^T
  constexpr int KT = BK / 32;  // 32-row key tiles of S^T
  constexpr int KC = BK / 16;  // 16-key chunks (contraction of O^T)
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int ROWB = D * 2;  // bytes per K/V row
  constexpr int LOADS = BK * CPR / kThreads;  // 16-byte slots per thread per tile
  static_assert(LOADS * kThreads == BK * CPR, "tile split");
  // With a bias (d <= 128) each wave streams its bias rows through a ring of
  // two tiles in LDS, and every direct load of the key loop is issued and
  // waited for by hand (see the pipeline below).  At d = 64 the K/V pipeline
  // gives up one stage for the ring, so two workgroups still fit a CU.
  constexpr bool kCounted =
      BIAS ? D <= 128
           : (FA_FWD_COUNTED && !SPLITKV && (D <= 128 || FA_FWD256_COUNTED));
  constexpr bool kBiasLds = BIAS && kCounted;
  constexpr int kStages = (kBiasLds && D == 64) ? 3 : FwdCfg<D>::STAGES;
  static_assert(kStages == 3 || kStages == 4, "the pipeline below runs three or four stages");
  static_assert(!kBiasLds || (QB == 1 && FwdCfg<D>::PREFETCH), "bias ring: one query block, score prefetch");
  // Pinned operand reads (d = 128) run FA_FWD_PIN_LA MFMAs ahead; with the
  // bias ring two ahead, which keeps every bias instantiation free of spills
  // (four ahead spilled 1-9 VGPRs in the causal, bf16 and fp32-output ones).
  constexpr int kPinLA = kCounted ? 2 : FA_FWD_PIN_LA;
  constexpr bool Q_LDS = FwdCfg<D>::Q_LDS;
  static_assert(!Q_LDS || QB == 1, "LDS-resident Q assumes one query block per wave");
  static_assert(!FwdCfg<D>::PIN || QB == 1, "pinned reads count one K read per MFMA");

  __shared__ __attribute__((aligned(16))) uint16_t sK[kStages][BK * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kStages][BK * D];
  // the workgroup's Q tile, row-major and swizzled like K (Q_LDS only)
  __shared__ __attribute__((aligned(16))) uint16_t sQ[Q_LDS ? BQ * D : 8];
  // bias ring: wave w, slot t % 2 holds its 32 rows x BK keys of tile t
  __shared__ __attribute__((aligned(16))) uint16_t sB[kBiasLds ? kWaves * 2 * 32 * BK : 8];

  const int tid = threadIdx.x;
  // (wave-uniform for the LDS-resident Q path, which then addresses its DMA
  // bases from scalar registers; the other paths measured better without)
  const int wave = Q_LDS ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 31;
  const int h = lane >> 5;

  int bh, qt, split = 0;
  {
    const int bid = blockIdx.x;
    const int S = SPLITKV ? a.splits : 1;
    if (CAUSAL) {
      qt = a.n_qtiles - 1 - bid / (a.BH * S);
      const int rem = bid % (a.BH * S);
      bh = rem / S;
      split = rem % S;
    } else {
      const int G = gridDim.x;
      const int lin = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
      const int item = a.item_base + lin / S;
      bh = item / a.n_qtiles;
      qt = item % a.n_qtiles;
      split = lin % S;
    }
  }
  const int N = a.N;
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const brsrc_t rq = make_rsrc(a.q + base, head_bytes);
  const brsrc_t rk = make_rsrc(a.k + base, head_bytes);
  const brsrc_t rv = make_rsrc(a.v + base, head_bytes);
  const int qw0 = qt * BQ + wave * (QB * 32);  // first query row of this wave
  // Attention bias rows of this head (N*N*2 < 2^32 is checked by the API).
  const brsrc_t rb =
      make_rsrc(BIAS ? a.bias + (bh / a.H) * a.bias_sb + (bh % a.H) * a.bias_sh : a.q,
                BIAS ? (uint32_t)N * N * 2 : 0u);
  // resource words and LDS addresses of the hand-counted loads (bias ring
  // only; LDS addresses are formed as 32-bit integers from the arrays
  // themselves, never through generic pointers)
  u32x4 wk{}, wv{}, wb{};
  const uint32_t lds_k = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&sK[0][0];
  const uint32_t lds_v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&sV[0][0];
  const uint32_t lds_b = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&sB[0];
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (kCounted) {
    wk = rsrc_words(a.k + base, head_bytes);
    wv = rsrc_words(a.v + base, head_bytes);
  }
  if constexpr (kBiasLds)
    wb = rsrc_words(a.bias + (bh / a.H) * a.bias_sb + (bh % a.H) * a.bias_sh, (uint32_t)N * N * 2);

  // Q^T fragments (B operand of S^T = K Q^T): lane (query m, half h), slot i
  // holds d = 16*dc + 8*h + i.  Rows past N read as 0.  With Q_LDS they are
  // read from sQ on every key tile instead (q_rd: this lane's chunk offsets in
  // its wave's 32 rows; rows are 16-byte-chunk swizzled so the 16 lanes of a
  // read cycle hit distinct bank slots).
  // The swizzles permute 16-byte chunks only within a 256-byte bank window,
  // so a lane's offsets repeat every window along a row: keep one window's
  // worth (RDC chunk pairs, RDT d tiles) and add the window offset as an
  // immediate.
  constexpr int RDC = DC < 8 ? DC : 8;
  constexpr int RDT = DT < 4 ? DT : 4;
  u32x4 qf[Q_LDS ? 1 : QB][Q_LDS ? 1 : DC];
  int q_rd[Q_LDS ? RDC : 1];
  if constexpr (Q_LDS) {
#pragma unroll
    for (int dc = 0; dc < RDC; ++dc)
      q_rd[dc] = ((wave * 32 + m) * D + (((2 * dc + h) ^ swz_dual<D>(m)) * 8)) * 2;
    // direct loads of the Q tile: slot p = i*256 + tid is tile row p / CPR at
    // chunk position p % CPR (global chunk (p % CPR) ^ swz(row))
    constexpr int QLOADS = BQ * CPR / kThreads;
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int p = i * kThreads + tid;
      const int row = p / CPR, cpos = p % CPR;
      const uint32_t voff = (uint32_t)(row * ROWB + ((cpos ^ swz_dual<D>(row)) * 16));
      if constexpr (kCounted) {
        bload16_lds_asm(rsrc_words(a.q + base, head_bytes),
                        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&sQ[0] +
                            (uint32_t)((i * kThreads + wave * 64) * 16),
                        voff, (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)qt * (uint32_t)(BQ * ROWB))));
      } else {
        bload16_lds(rq, (char*)sQ + (i * kThreads + wave * 64) * 16, voff, (uint32_t)qt * (uint32_t)(BQ * ROWB));
      }
    }
  } else {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        qf[qb][dc] = bload16(rq, ((uint32_t)(qw0 + qb * 32 + m) * D + dc * 16 + 8 * h) * 2u, 0);
  }

  // K operand (A of S^T): row kt*32 + perm_k(m), chunk 2dc+h, swizzled.
  int k_rd[RDC];
  {
    const int row = perm_k(m);
#pragma unroll
    for (int dc = 0; dc < RDC; ++dc) k_rd[dc] = (row * D + (((2 * dc + h) ^ swz_dual<D>(row)) * 8)) * 2;
  }
  auto k_off = [&](int dc) { return k_rd[dc % RDC] + (dc / RDC) * 256; };
  auto q_off = [&](int dc) { return q_rd[dc % RDC] + (dc / RDC) * 256; };
  // V^T operand (A of O^T) through the transposing read.  In 16-lane group g
  // (gg = g % 2), lane i = 4j + q reads key 8h + 4r + j (r: which half of the
  // 8 k-slots) at the 4-element d quad dquad(gg, q) = 16(q%2) + 8gg + 4(q/2)
  // of d tile dt; lane i then receives d = perm_o(16gg + i) for 4 keys.
  int v_tr[RDT];
  {
    const int i = lane & 15, gg = (lane >> 4) & 1;
    const int j = i >> 2, q = i & 3;
#pragma unroll
    for (int dt = 0; dt < RDT; ++dt) {
      const int chunk = 4 * dt + 2 * (q & 1) + gg;
      v_tr[dt] = (8 * h + j) * ROWB + ((chunk ^ swz_tr<D>(j)) * 16) + (q >> 1) * 8;
    }
  }
  auto v_off = [&](int dt) { return v_tr[dt % RDT] + (dt / RDT) * 256; };
  // With the bias ring at d = 64 the compiler places the V array 64 KB or
  // more into LDS, beyond a read's 16-bit offset field, and then adds the
  // array's address with a VALU op before every read.  Those kernels keep the
  // address in the per-lane bases (hidden from the compiler) instead.
  constexpr bool kVBase = kBiasLds && D == 64;
  uint32_t v_ta[kVBase ? RDT : 1];
  if constexpr (kVBase) {
#pragma unroll
    for (int dt = 0; dt < RDT; ++dt) {
      v_ta[dt] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&sV[0][0] + (uint32_t)v_tr[dt];
      asm volatile("" : "+v"(v_ta[dt]));
    }
    static_assert((kStages - 1) * BK * ROWB + (DT / RDT - 1) * 256 + (KC - 1) * 16 * ROWB + 4 * ROWB + 8 < 65536,
                  "V read constants fit the offset field");
  }
  // V^T operand of d tile dt and 16-key chunk kc from the stage at Vb
  auto v_read = [&](const char* Vb, int dt, int kc, u32x2& lo, u32x2& hi) {
    if constexpr (kVBase) {
      const uint32_t at = v_ta[dt % RDT] + (uint32_t)(Vb - (const char*)&sV[0][0]) +
                          (uint32_t)((dt / RDT) * 256 + kc * 16 * ROWB);
      lo = lds_read_tr16_at(at);
      hi = lds_read_tr16_at(at + 4 * ROWB);
    } else {
      lo = lds_read_tr16(Vb + v_off(dt) + kc * 16 * ROWB);
      hi = lds_read_tr16(Vb + v_off(dt) + kc * 16 * ROWB + 4 * ROWB);
    }
  };
  // Direct-load slots: thread slot p = i*256 + tid holds tile row p / CPR at
  // swizzled chunk position p % CPR, i.e. global chunk (p % CPR) ^ swz(row).
  uint32_t k_gl[LOADS], v_gl[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = i * kThreads + tid;
    const int row = p / CPR, cpos = p % CPR;
    k_gl[i] = (uint32_t)(row * ROWB + ((cpos ^ swz_dual<D>(row)) * 16));
    v_gl[i] = (uint32_t)(row * ROWB + ((cpos ^ swz_tr<D>(row)) * 16));
  }

  const int kend = CAUSAL ? min(N, qt * BQ + BQ) : N;
  // This workgroup's key tiles: j0 .. j0 + n_kt - 1 (all of them unless split).
  int j0 = 0, n_kt = (kend + BK - 1) / BK;
  if constexpr (SPLITKV) {
    const int total = n_kt;
    j0 = (int)(((long long)split * total) / a.splits);
    n_kt = (int)(((long long)(split + 1) * total) / a.splits) - j0;
  }

  // `live` false: a tile past the end, loaded from past the resource (zeros,
  // no memory traffic) so that the number of loads in flight stays fixed.
  auto issue_tile = [&](int j, uint16_t* dk, uint16_t* dv, bool live = true) {
    if constexpr (kCounted) {
      const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(live ? (uint32_t)(j0 + j) * (uint32_t)(BK * ROWB) : head_bytes));
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t off = (uint32_t)(((dk - &sK[0][0]) * 2) + (i * kThreads + wave_u * 64) * 16);
        bload16_lds_asm(wk, lds_k + off, k_gl[i], soff);
        bload16_lds_asm(wv, lds_v + off, v_gl[i], soff);
      }
    } else {
      const uint32_t soff = (uint32_t)(j0 + j) * (uint32_t)(BK * ROWB);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        char* kb = (char*)dk + (i * kThreads + wave * 64) * 16;
        char* vb = (char*)dv + (i * kThreads + wave * 64) * 16;
        bload16_lds(rk, kb, k_gl[i], soff);
        bload16_lds(rv, vb, v_gl[i], soff);
      }
    }
  };

  // Bias ring.  A wave's tile block is 32 rows x BK keys, row-major, with the
  // 16-byte chunks of row r at positions chunk ^ swz_b(r): 16 lanes reading
  // one chunk of 16 consecutive rows then hit distinct bank slots of the
  // 256-byte window.  Direct load i, lane l fills slot 64i + l, i.e. row
  // (64i + l) / CPRB at position (64i + l) % CPRB.
  constexpr int CPRB = BK / 8;           // 16-byte chunks per bias row of a tile
  constexpr int RPW = 256 / (BK * 2);    // bias rows per 256-byte window
  constexpr int LB = 32 * CPRB / 64;     // direct loads per lane per tile
  auto swz_b = [](int row) { return (row / RPW) % CPRB; };
  uint32_t b_gl[kBiasLds ? LB : 1];
  if constexpr (kBiasLds) {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int p = i * 64 + lane;
      const int row = p / CPRB, pos = p % CPRB;
      b_gl[i] = (uint32_t)(qw0 + row) * (uint32_t)N * 2u + (uint32_t)((pos ^ swz_b(row)) * 16);
    }
  }
  auto bias_slot = [&](int t) { return sB + (wave * 2 + (t & 1)) * 32 * BK; };
  auto issue_bias = [&](int t, bool live) {
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(live ? (uint32_t)(j0 + t) * (uint32_t)(BK * 2) : (uint32_t)N * (uint32_t)N * 2u));
    const uint32_t slot = lds_b + (uint32_t)((wave_u * 2 + (t & 1)) * 32 * BK * 2);
#pragma unroll
    for (int i = 0; i < LB; ++i) bload16_lds_asm(wb, slot + i * 64 * 16, b_gl[i], soff);
  };

  // m_run: exponent reference (log2 units); l_run: sum of the rounded
  // probabilities (normalises O); l32_run: fp32 sum for the bf16 LSE.
  float m_run[QB], l_run[QB], l32_run[QB];
  f32x16 oacc[QB][DT];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
    l32_run[qb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qb][dt] = f32x16{};
  }

  const float c = a.c;

  // s + bias / scale, so that c * (s + bias/scale) = c*s + bias*log2(e);
  // applied before the mask, which then overrides whatever the bias read
  // past the end of a row.  ab[qb][kt][g] holds this lane's bias for keys
  // 32kt + 16g + 8h + 0..7 of the tile.
  auto add_bias = [&](f32x16 (&s)[QB][KT], const u32x4 (&ab)[QB][KT][2]) {
    const float kb = kLog2e / c;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = ab[qb][kt][g][e];
            s[qb][kt][8 * g + 2 * e] =
                __builtin_fmaf(to_f32<BF16>((uint16_t)(w & 0xffffu)), kb, s[qb][kt][8 * g + 2 * e]);
            s[qb][kt][8 * g + 2 * e + 1] =
                __builtin_fmaf(to_f32<BF16>((uint16_t)(w >> 16)), kb, s[qb][kt][8 * g + 2 * e + 1]);
          }
  };

  // S^T = K Q^T for one K tile (the scores of 32*KT keys against this wave's
  // query blocks), and with an attention bias its raw bias values: register
  // group g = r/8 of key block kt holds keys k_first + 32kt + 16g + 8h + 0..7,
  // eight consecutive entries of this lane's bias row (one 16-byte load).
  struct Scores {
    f32x16 v[QB][KT];
    u32x4 ab[QB][KT][2];
  };
  auto compute_scores = [&](const uint16_t* Ks, int k_first) {
    const char* Kb = (const char*)Ks;
    Scores sc;
    if constexpr (BIAS && !kBiasLds) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int g = 0; g < 2; ++g)
            sc.ab[qb][kt][g] = bload16(
                rb, ((uint32_t)(qw0 + qb * 32 + m) * (uint32_t)N + (uint32_t)(k_first + 32 * kt + 16 * g + 8 * h)) * 2u, 0);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) sc.v[qb][kt] = f32x16{};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4 af = *(const u32x4*)(Kb + kt * 32 * ROWB + k_off(dc));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if constexpr (Q_LDS) {
            const u32x4 bq = *(const u32x4*)((const char*)sQ + q_off(dc));
            sc.v[qb][kt] = mfma32<BF16>(af, bq, sc.v[qb][kt]);
            pin_step<1, 2, FA_QLDS_LOOKAHEAD>(kt * DC + dc);
          } else {
            sc.v[qb][kt] = mfma32<BF16>(af, qf[qb][dc], sc.v[qb][kt]);
            if constexpr (FwdCfg<D>::PIN) pin_step<1, 1, kPinLA>(kt * DC + dc);
          }
        }
      }
    if constexpr (Q_LDS) pin_tail<1, FA_QLDS_LOOKAHEAD>();
    if constexpr (FwdCfg<D>::PIN) pin_tail<1, kPinLA>();
    return sc;
  };

  // Online softmax of one tile's scores and O^T += V^T P^T.  MASK: apply the
  // causal diagonal and the end of the sequence (only on tiles that straddle
  // them).
  // `issue_next` issues the score MFMAs of the following tile; it is called
  // once on every path, inside the same basic block as this tile's
  // exponentials, so the scheduler can interleave the two.
  auto softmax_pv = [&](auto mask_tag, Scores& sc, const uint16_t* Vs, int k0, bool first,
                        auto&& issue_next) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* Vb = (const char*)Vs;
    auto& s = sc.v;
    if constexpr (BIAS && !kBiasLds) add_bias(s, sc.ab);

    // O^T += V^T P^T for packed probabilities pf.
    auto pv = [&](const u32x4 (&pf)[QB][KC]) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          u32x2 lo, hi;
          v_read(Vb, dt, kc, lo, hi);
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][dt] = mfma32<BF16>(vf, pf[qb][kc], oacc[qb][dt]);
          if constexpr (Q_LDS) pin_step<2, 2, FA_QLDS_LOOKAHEAD>(dt * KC + kc);
          if constexpr (FwdCfg<D>::PIN) pin_step<2, 2, kPinLA>(dt * KC + kc);
        }
      if constexpr (Q_LDS) pin_tail<2, FA_QLDS_LOOKAHEAD>();
      if constexpr (FwdCfg<D>::PIN) pin_tail<2, kPinLA>();
    };
    if constexpr (!BF16) {
      // ---- fp16: lazy reference, overflow detected from the rounded sum ----
      if constexpr (MASK) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qrow = qw0 + qb * 32 + m;
          const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;  // last visible key
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
              if (key > lim) s[qb][kt][r] = -INFINITY;
            }
        }
      }
      // p = 2^(c*s - m_run) rounded to fp16, packed as the P^T operand;
      // tsum: this lane's sum of the rounded values.
      auto exp_pack = [&](int qb, u32x4 (&pfq)[KC], float& tsum) {
        const float neg_m = -m_run[qb];
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * half + 2 * e;
              const float x0 = __builtin_fmaf(s[qb][kt][r], c, neg_m);
              const float x1 = __builtin_fmaf(s[qb][kt][r + 1], c, neg_m);
              w[e] = pack2<false>(fast_exp2(x0), fast_exp2(x1));
              if (e & 1) t1 = sum2<false>(w[e], t1); else t0 = sum2<false>(w[e], t0);
            }
            pfq[2 * kt + half] = w;
          }
        tsum = t0 + t1;
      };
      // Exact path: rows that need it (need[qb]: first tile, or this row's
      // rounded sum left the safe range) raise the reference to the row max
      // where the max exceeds it (first tile: set it to the row max) and
      // rescale; every row then exponentiates again.  Rows that did not need
      // it keep their reference and recompute identical values, so each row
      // depends on its own data alone.
      auto slow = [&](const bool (&need)[QB]) {
        u32x4 pf[QB][KC];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
              mx0 = fmaxf(mx0, fmaxf(s[qb][kt][r], s[qb][kt][r + 1]));
              mx1 = fmaxf(mx1, fmaxf(s[qb][kt][r + 2], s[qb][kt][r + 3]));
            }
          const float mx = max_halves(fmaxf(mx0, mx1)) * c;
          float m_new = first ? mx : fmaxf(m_run[qb], mx);
          if (!need[qb]) m_new = m_run[qb];
          // A row with no visible key so far (a bias can hide whole tiles, a
          // split can start past a causal row) takes a finite reference below
          // any score: its probabilities are 0 now, and on the first tile with
          // a visible key every fast-path exponent overflows, so that row
          // takes this exact path again and sets its reference to the row max.
          if (m_new == -INFINITY) m_new = kNoReference;
          if (!first) {
            const float alpha = fast_exp2(m_run[qb] - m_new);
            l_run[qb] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[qb][dt] *= alpha;
          }
          m_run[qb] = m_new;
          float ts;
          exp_pack(qb, pf[qb], ts);
          l_run[qb] += ts;
        }
        pv(pf);
      };
      if (first) {
        issue_next();
        bool need[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) need[qb] = first;
        slow(need);
      } else {
        // Fast path: keep the reference while the row's rounded tile sum stays
        // at or below 2^12 (so every probability does, far from fp16
        // overflow); a larger sum, an infinity or a new max more than 12
        // (log2 units) above the reference takes the exact path.
        // Non-causal launches raise the wave's issue priority for the next
        // tile's score MFMAs and this tile's exponentials, and drop it for
        // the P V product, so that the two waves sharing a SIMD tend to
        // alternate between the phases (measured -2% at B2 H12 N8192; the
        // causal instantiation measured +6% and keeps the default).
        if constexpr (kPrioScores > 0 && !CAUSAL) __builtin_amdgcn_s_setprio(kPrioScores);
        issue_next();
        u32x4 pf[QB][KC];
        float ts[QB];
        bool need[QB];
        bool big = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          exp_pack(qb, pf[qb], ts[qb]);
          // both halves of the wave hold parts of the same rows: decide on the
          // row's sum so the two halves agree
          need[qb] = !(sum_halves(ts[qb]) <= kLazyBound);
          big = big || (__ballot(need[qb]) != 0ull);
        }
#if FA_FWD_SCHED_VALU > 0
        if constexpr (!Q_LDS) {
        // Interleave the next tile's score MFMAs with this tile's VALU work:
        // operand reads first, then one MFMA per group of VALU instructions.
        __builtin_amdgcn_sched_group_barrier(0x100, DC * KT, 0);
#pragma unroll
        for (int i = 0; i < QB * KT * DC; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, FA_FWD_SCHED_VALU, 0);
        }
        }
#endif
        if constexpr (kPrioScores > 0 && !CAUSAL) __builtin_amdgcn_s_setprio(0);
        // (marked unlikely where it measured faster: the non-causal kernels,
        // -0.6% at d=64 and -1.1% at d=128; the causal ones spilled with it)
        if (CAUSAL ? big : __builtin_expect(big, 0)) {
          slow(need);
        } else {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) l_run[qb] += ts[qb];
          pv(pf);
        }
      }
      return;
    }
    issue_next();
    if constexpr (MASK) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qrow = qw0 + qb * 32 + m;
        const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;  // last visible key
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
            if (key > lim) s[qb][kt][r] = -INFINITY;
          }
      }
    }
    // ---- online softmax --------------------------------------------------
    float mnew[QB];
    bool grow[QB];
    bool any_grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          mx0 = fmaxf(mx0, fmaxf(s[qb][kt][r], s[qb][kt][r + 1]));
          mx1 = fmaxf(mx1, fmaxf(s[qb][kt][r + 2], s[qb][kt][r + 3]));
        }
      mnew[qb] = max_halves(fmaxf(mx0, mx1)) * c;
      grow[qb] = mnew[qb] > m_run[qb] + rescale_threshold<BF16>();
      any_grow = any_grow || (__ballot(grow[qb]) != 0ull);
    }
    // Only rows that grew move their reference (the others get alpha = 1
    // exactly), so each row depends on its own data alone.
    auto rescale = [&](int qb) {
      const float mn = grow[qb] ? mnew[qb] : m_run[qb];
      const float alpha = (m_run[qb] == -INFINITY) ? 0.f : fast_exp2(m_run[qb] - mn);
      m_run[qb] = mn;
      l_run[qb] *= alpha;
      if constexpr (BF16) l32_run[qb] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[qb][dt] *= alpha;
    };
    // Exponentiate, round, sum and multiply by V^T.  Instantiated twice so
    // that the path without a rescale carries no merge copies of O.
    auto finish = [&](auto rescale_tag) {
      constexpr bool RESCALE = decltype(rescale_tag)::value;
      u32x4 pf[QB][KC];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (RESCALE) rescale(qb);
        const float neg_m = (m_run[qb] == -INFINITY) ? 0.f : -m_run[qb];
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
        float ls32[2] = {0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = fast_exp2(__builtin_fmaf(s[qb][kt][r], c, neg_m));
            if constexpr (BF16) ls32[r & 1] += p[r];
          }
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] = pack2<BF16>(p[8 * half + 2 * e], p[8 * half + 2 * e + 1]);
              ls[e] = sum2<BF16>(w[e], ls[e]);
            }
            pf[qb][2 * kt + half] = w;
          }
        }
        l_run[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        if constexpr (BF16) l32_run[qb] += ls32[0] + ls32[1];
      }
      // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          u32x2 lo, hi;
          v_read(Vb, dt, kc, lo, hi);
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][dt] = mfma32<BF16>(vf, pf[qb][kc], oacc[qb][dt]);
          if constexpr (Q_LDS) pin_step<2, 2, FA_QLDS_LOOKAHEAD>(dt * KC + kc);
          if constexpr (FwdCfg<D>::PIN) pin_step<2, 2, kPinLA>(dt * KC + kc);
        }
      if constexpr (Q_LDS) pin_tail<2, FA_QLDS_LOOKAHEAD>();
      if constexpr (FwdCfg<D>::PIN) pin_tail<2, kPinLA>();
    };
    // Causal d <= 128: rows whose max grew are rescaled in a block of their
    // own and the exponentials and P V run on one path.  With two
    // instantiated paths the allocator copied all of O (16 or 32 v_mov_b64
    // per tile) on the common, non-growing one; one path measured -5.0% at
    // B2 H16 N4096 d128 and -2.7% at B1 H8 N32768 d64 (bf16, causal).  The
    // non-causal d=128 and the d=256 instantiations spill or slow down with
    // one path (+1.8%, +30%) and keep two.
    if constexpr (CAUSAL && D <= 128) {
      if (any_grow) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) rescale(qb);
      }
      finish(std::false_type{});
    } else {
      if (any_grow) {
        finish(std::true_type{});
      } else {
        finish(std::false_type{});
      }
    }
  };

  // Software pipeline over K/V tiles, kStages LDS stages deep.  Iteration j
  // (tile j in stage j % kStages) starts the loads of tile j + kStages - 1
  // (into the stage tile j - 1 left), issues the score MFMAs of tile j + 1 -
  // independent of this tile's softmax, so the matrix cores have work while
  // the softmax runs on the VALU - then runs the softmax and P V of tile j.
  // Before the group barrier it waits until tile j + 2 has landed (needed by
  // the next iteration's scores).  Direct loads complete in issue order, so
  // this is "all but the newest kStages - 3 tiles".
  constexpr int kTileLoads = 2 * LOADS;  // direct loads per thread per tile
  constexpr int kAhead = kStages - 1;    // prefetch distance in tiles
  // Without the score prefetch (PREFETCH false) an iteration computes its own
  // tile's scores first and the next iteration needs only tile j + 1.
  constexpr bool PREFETCH = FwdCfg<D>::PREFETCH;
  constexpr int kKeep = (PREFETCH ? kStages - 3 : kStages - 2) * kTileLoads;
  // With the bias ring (kBiasLds) the iteration issues, in this order, tile
  // j + kAhead's K/V and tile j + 2's bias, both unconditionally (tiles past
  // the end load nothing), so the loads in flight follow a fixed pattern:
  //  * tile j's bias was issued after tile j - 2 + kAhead's K/V; newer than
  //    it when it is read are the K/V of two tiles and one tile's bias;
  //  * at the end of iteration j tile j + 2's K/V must have landed (the next
  //    iteration computes its scores); newer than it are kAhead - 2 tiles of
  //    K/V and kAhead - 1 tiles of bias.
  // The compiler sees none of these loads, so it adds no waits of its own.
  constexpr int LBc = kBiasLds ? LB : 0;  // bias loads per tile in the count
  constexpr int kBiasKeepRead = 2 * kTileLoads + LBc;
  constexpr int kCountedKeepEnd = (kAhead - 2) * kTileLoads + (kAhead - 1) * LBc;
  // CLEAN: a tile below the causal diagonal for every row of the workgroup
  // and inside N, compiled with neither the mask nor the active check.
  auto iteration = [&](int j, auto stage_tag, Scores& cur, Scores& nxt, auto clean_tag) {
    constexpr int st = decltype(stage_tag)::value;
    constexpr bool CLEAN = decltype(clean_tag)::value;
    if constexpr (kBiasLds) {
      issue_tile(j + kAhead, sK[(st + kAhead) % kStages], sV[(st + kAhead) % kStages], j + kAhead < n_kt);
    } else {
      if (j + kAhead < n_kt)
        issue_tile(j + kAhead, sK[(st + kAhead) % kStages], sV[(st + kAhead) % kStages]);
    }
    // On the last tile this reads a stale (in-bounds) stage whose scores are
    // never used; keeping it unconditional keeps it in one basic block with
    // the exponentials.
    auto issue_next = [&]() {
      if constexpr (PREFETCH) nxt = compute_scores(sK[(st + 1) % kStages], (j0 + j + 1) * BK);
    };
    const int k0 = (j0 + j) * BK;
    const bool active = CLEAN || !CAUSAL || (k0 <= qw0 + QB * 32 - 1);
    if constexpr (kBiasLds) {
      wait_vmem_keep<kBiasKeepRead>();  // this tile's bias has landed
      if (active) {
        const char* bb = (const char*)bias_slot(j);
        u32x4 ab[QB][KT][2];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int g = 0; g < 2; ++g)
            ab[0][kt][g] = *(const u32x4*)(bb + m * (BK * 2) + (((4 * kt + 2 * g + h) ^ swz_b(m)) * 16));
        add_bias(cur.v, ab);
      }
      wait_lds();  // (the slot's reads have returned before it is refilled)
      issue_bias(j + 2, j + 2 < n_kt);
    }
    if (active) {
      if constexpr (!PREFETCH) cur = compute_scores(sK[st], k0);
      const bool need_mask = !CLEAN && ((k0 + BK > N) || (CAUSAL && k0 + BK - 1 > qw0));
      if (need_mask) {
        softmax_pv(std::true_type{}, cur, sV[st], k0, j == 0, issue_next);
      } else {
        softmax_pv(std::false_type{}, cur, sV[st], k0, j == 0, issue_next);
      }
    } else {
      issue_next();
    }
    if constexpr (kBiasLds) {
      wait_vmem_keep<kCountedKeepEnd>();
      barrier_no_fence();
    } else {
      // (without a bias no load is issued past the end, so the last kAhead
      // iterations wait for everything)
      if (j + kAhead < n_kt) {
        wait_vmem_keep<kKeep>();
      } else {
        wait_vmem();
      }
      if constexpr (kCounted) {
        barrier_no_fence();
      } else {
        __syncthreads();
      }
    }
  };

  // (with Q_LDS the Q tile's loads were issued first, so they land first)
  if constexpr (kBiasLds) {
    // tile 0's bias, K/V of tiles 0 .. kAhead - 1, tile 1's bias: from tile
    // 1 on, each bias follows the K/V of the tile kAhead - 2 after it, as in
    // the loop; wait for tiles 0 and 1 (and so for tile 0's bias)
    issue_bias(0, true);
#pragma unroll
    for (int s0 = 0; s0 < kAhead; ++s0) issue_tile(s0, sK[s0], sV[s0], s0 < n_kt);
    issue_bias(1, 1 < n_kt);
    wait_vmem_keep<(kAhead - 2) * kTileLoads + LB>();
    barrier_no_fence();
  } else {
#pragma unroll
    for (int s0 = 0; s0 < kAhead; ++s0)
      if (s0 < n_kt) issue_tile(s0, sK[s0], sV[s0]);
  if (kAhead < n_kt) {
    wait_vmem_keep<kKeep>();  // tiles 0 and 1 (without the prefetch: tile 0) have landed
  } else {
    wait_vmem();
  }
  __syncthreads();
  }
  Scores sa, sb;
  if constexpr (PREFETCH) sa = compute_scores(sK[0], j0 * BK);
  int j = 0;
  // Whole rounds of tiles that lie below the diagonal for every row of the
  // workgroup (global tile t with (t + 1) BK - 1 <= qt BQ) and inside N run a
  // loop body without masks or active checks.  Measured (same box, outputs
  // bit-identical): bf16 d=64 causal -2.6% (B1 H8 N32768) and -3.7% (B2 H12
  // N4096), fp16 d=128 causal -1.8%; fp16 d=64 causal +1.9% with the
  // compiler's load waits and -2.5 to -9% (+0.7% at B2 H12 N4096) with the
  // hand-counted ones, which it now takes.  The bias kernels (not measured)
  // and the split-KV ones (where the second body cost a spilled register)
  // keep the single loop.
  constexpr bool kCleanLoop = CAUSAL && !BIAS && !SPLITKV && D <= 128;
  if constexpr (kCleanLoop) {
    const int n_clean = min(n_kt, max(0, min((qt * BQ + 1) / BK, N / BK) - j0));
    for (; j + kStages <= n_clean; j += kStages) {
      iteration(j, std::integral_constant<int, 0>{}, sa, sb, std::true_type{});
      iteration(j + 1, std::integral_constant<int, 1>{}, sb, sa, std::true_type{});
      iteration(j + 2, std::integral_constant<int, 2>{}, sa, sb, std::true_type{});
      if constexpr (kStages == 4) {
        iteration(j + 3, std::integral_constant<int, 3>{}, sb, sa, std::true_type{});
      } else if constexpr (PREFETCH) {
        sa = sb;
      }
    }
  }
  for (; j < n_kt; j += kStages) {
    iteration(j, std::integral_constant<int, 0>{}, sa, sb, std::false_type{});
    if (j + 1 < n_kt) iteration(j + 1, std::integral_constant<int, 1>{}, sb, sa, std::false_type{});
    if (j + 2 < n_kt) iteration(j + 2, std::integral_constant<int, 2>{}, sa, sb, std::false_type{});
    if constexpr (kStages == 4) {
      if (j + 3 < n_kt) iteration(j + 3, std::integral_constant<int, 3>{}, sb, sa, std::false_type{});
    } else if constexpr (PREFETCH) {
      sa = sb;  // an odd number of tiles per round: the next round starts from sb
    }
  }
  // (the ring's loads past the end are still in flight: let them land before
  // the workgroup's LDS can be handed to another)
  if constexpr (kBiasLds) wait_vmem();

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
  // A row that saw no key (only possible in a split) has l = 0: O = 0 and
  // LSE = -inf, which the split merge weights by zero.
  if constexpr (SPLITKV) {
    // this work item's rows r0 .. r0 + cnt - 1 of the head, as partial rows
    const int r0 = qt * BQ, cnt = min(BQ, N - r0);
    const size_t prow = (size_t)split * a.part_rows + (size_t)bh * N + r0 - a.part_row_base;
    const brsrc_t ro = make_rsrc(a.part_o + prow * D, (uint32_t)cnt * D * 4);
    const brsrc_t rl = make_rsrc(a.part_lse + prow, (uint32_t)cnt * 4);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = qw0 + qb * 32 + m - r0;
      const float lt = sum_halves(l_run[qb]);
      const float ll = BF16 ? sum_halves(l32_run[qb]) : lt;
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int col = dt * 32 + 16 * h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = __float_as_uint(oacc[qb][dt][4 * e + t] * inv);
          bstore16(w, ro, ((uint32_t)row * D + col + 4 * e) * 4u, 0);
        }
      }
      if (h == 0)
        bstore4(ll > 0.f ? (m_run[qb] + fast_log2(ll)) * kLn2 : -INFINITY, rl, (uint32_t)row * 4u, 0);
    }
    return;
  }
  const brsrc_t ro = make_rsrc((const char*)a.o + base * (OUT_F32 ? 4 : 2),
                               (uint32_t)N * D * (OUT_F32 ? 4 : 2));
  const brsrc_t rl = make_rsrc(a.lse + (size_t)bh * N, (uint32_t)N * 4);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + m;  // rows past N are dropped by the stores
    const float lt = sum_halves(l_run[qb]);
    const float ll = BF16 ? sum_halves(l32_run[qb]) : lt;
    // a bias can hide every key of a row: then O = 0 and LSE = -inf
    const float inv = (!BIAS || lt > 0.f) ? 1.0f / lt : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int col = dt * 32 + 16 * h;
      if constexpr (OUT_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = __float_as_uint(oacc[qb][dt][4 * e + t] * inv);
          bstore16(w, ro, ((uint32_t)row * D + col + 4 * e) * 4u, 0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          u32x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            w[t] = pack2<BF16>(oacc[qb][dt][8 * e + 2 * t] * inv, oacc[qb][dt][8 * e + 2 * t + 1] * inv);
          bstore16(w, ro, ((uint32_t)row * D + col + 8 * e) * 2u, 0);
        }
      }
    }
    if (h == 0)
      bstore4((!BIAS || ll > 0.f) ? (m_run[qb] + fast_log2(ll)) * kLn2 : -INFINITY, rl,
              (uint32_t)row * 4u, 0);
  }
}

// Split-KV merge (one pass over the partial results): per row,
// LSE = logsumexp_s LSE_s and O = sum_s exp(LSE_s - LSE) O_s.  Splits whose
// range held no visible key carry LSE_s = -inf and weigh nothing.
template <int D, bool BF16, bool OUT_F32>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const float* part_o, const float* part_lse,
                                                       void* o, float* lse, int rows, int splits) {
  constexpr int L = D / 4;        // lanes per row, four values each
  constexpr int RPB = 256 / L;    // rows per workgroup
  const int row = blockIdx.x * RPB + (int)threadIdx.x / L;
  const int col = ((int)threadIdx.x % L) * 4;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, part_lse[(size_t)s * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float w = fast_exp2((part_lse[(size_t)s * rows + row] - mx) * kLog2e);
      const f32x4 x = *(const f32x4*)(part_o + ((size_t)s * rows + row) * D + col);
      wsum += w;
      acc += w * x;
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  acc *= inv;
  if constexpr (OUT_F32) {
    *(f32x4*)((float*)o + (size_t)row * D + col) = acc;
  } else {
    u32x2 w2 = {pack2<BF16>(acc[0], acc[1]), pack2<BF16>(acc[2], acc[3])};
    *(u32x2*)((uint16_t*)o + (size_t)row * D + col) = w2;
  }
  if (col == 0) lse[row] = wsum > 0.f ? mx + fast_log2(wsum) * kLn2 : -INFINITY;
}

template <int D, bool BF16, bool CAUSAL, bool OUT_F32, bool SPLITKV, bool BIAS>
hipError_t launch_fwd_t(const FwdProblem& p, hipStream_t stream) {
  constexpr int BQ = kWaves * FwdCfg<D>::QB * 32;
  FwdArgs a;
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.o = p.o;
  a.lse = p.lse;
  a.N = p.N;
  a.BH = p.BH;
  a.n_qtiles = (p.N + BQ - 1) / BQ;
  a.c = p.scale * kLog2e;
  a.splits = SPLITKV ? p.splits : 1;
  a.part_row_base = SPLITKV ? p.part_row_base : 0;
  a.part_rows = SPLITKV ? (p.part_rows > 0 ? p.part_rows : p.BH * p.N) : 0;
  a.part_o = SPLITKV ? p.part : nullptr;
  a.part_lse = SPLITKV ? p.part + (size_t)p.splits * a.part_rows * D : nullptr;
  a.item_base = p.item_base;
  const int n_items = p.item_count > 0 ? p.item_count : a.BH * a.n_qtiles - p.item_base;
  a.bias = (const uint16_t*)p.bias;
  a.bias_sb = p.bias_sb;
  a.bias_sh = p.bias_sh;
  a.H = p.H;
  const dim3 grid((unsigned)(n_items * a.splits));
  hipLaunchKernelGGL((fwd_kernel<D, BF16, CAUSAL, OUT_F32, SPLITKV, BIAS>), grid, dim3(kThreads), 0,
                     stream, a);
  if (!SPLITKV) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // merge the partial rows into rows part_row_base .. of O and LSE
  const int rows = a.part_rows;
  constexpr int RPB = 256 / (D / 4);
  void* o_rows = (char*)p.o + (size_t)a.part_row_base * D * (OUT_F32 ? 4 : 2);
  hipLaunchKernelGGL((fwd_merge_kernel<D, BF16, OUT_F32>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                     dim3(256), 0, stream, a.part_o, a.part_lse, o_rows, p.lse + a.part_row_base, rows,
                     p.splits);
  return hipGetLastError();
}

template <int D, bool BF16, bool OUT_F32, bool SPLITKV, bool BIAS>
hipError_t launch_fwd_c(const FwdProblem& p, hipStream_t s) {
  return p.causal ? launch_fwd_t<D, BF16, true, OUT_F32, SPLITKV, BIAS>(p, s)
                  : launch_fwd_t<D, BF16, false, OUT_F32, SPLITKV, BIAS>(p, s);
}

template <int D, bool SPLITKV, bool BIAS>
hipError_t launch_fwd_d(const FwdProblem& p, hipStream_t s) {
  switch (p.dtype) {
    case kF16: return launch_fwd_c<D, false, false, SPLITKV, BIAS>(p, s);
    case kBF16: return launch_fwd_c<D, true, false, SPLITKV, BIAS>(p, s);
    case kF16OutF32: return launch_fwd_c<D, false, true, SPLITKV, BIAS>(p, s);
    case kBF16OutF32: return launch_fwd_c<D, true, true, SPLITKV, BIAS>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
