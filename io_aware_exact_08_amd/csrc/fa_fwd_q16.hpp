// Fused exact-attention forward for head dimensions 128 and 256 on 16x16x32
// MFMAs with 16-query waves.
//
// The method is fwd_kernel's (page 2 of the subject, "Kernel Fusion" and
// "Tiling": scores, online softmax and P V per tile, one normalisation at the
// end, O and the row LSE written once).  What changes is the mapping, chosen
// so that the registers of a wave shrink (two waves fit each SIMD at d = 256):
//  * A workgroup is 8 waves of 16 query rows each, 128 rows in all.  At
//    d = 256 a wave's O^T (256 d x 16 queries) is 16 accumulator tiles of four
//    registers, 64 in all, and its Q^T operand 32 registers; with 32 queries
//    per wave (fwd_kernel) O alone takes 128 and the accumulators had to be
//    parked in the accumulation registers around every product.  At d = 128
//    both halve.
//  * S^T = K Q^T per 16-key block with v_mfma_f32_16x16x32: lane l holds
//    query l%16 and keys 4(l/16) .. 4(l/16)+3 of the block.  A row's 32 keys
//    of a tile sit in lanes l%16 + 16g, g = 0..3, so its max and sum combine
//    over those four lanes (ds_swizzle for the xor-16 pair, permlane32_swap
//    for the halves).  Every O register of a lane belongs to its query, so a
//    rescale multiplies the lane's accumulators by one factor, and the row
//    max is cheap enough to take on every tile (one exponential/P V path for
//    both input types).
//  * The lane's eight probabilities of a tile (keys 4g+j and 16+4g+j, j < 4)
//    are exactly the eight k-slots it supplies to O^T += V^T P^T; the V^T
//    operand is read with ds_read_b64_tr_b16 from the same two groups of four
//    keys, so P goes from the score registers to the next product directly.
//  * K and V tiles of 32 keys stream through four LDS stages (128 KB at
//    d = 256, 64 KB at d = 128) by direct buffer->LDS loads that the kernel
//    counts itself (the compiler would otherwise wait for all of them before
//    every LDS read).  K rows are swizzled so that the 16 lanes reading one
//    chunk of 16 consecutive rows hit 16 bank slots; V rows so that the
//    transposing read's 32 lanes of a cycle (8 rows x 2 chunks) do.  Both
//    XORs stay inside a 256-byte bank window, which a row fills at d = 128
//    and half fills at d = 256.
#pragma once

#include "fa_fwd.hpp"

namespace fa {

constexpr int kWQ16 = 8;              // waves per workgroup
constexpr int kTQ16 = kWQ16 * 64;     // threads
constexpr int kBQQ16 = kWQ16 * 16;    // query rows per workgroup
constexpr int kBKQ16 = 32;            // keys per tile
constexpr int kStQ16 = 4;             // LDS stages
static_assert(kBQQ16 == kWaves * FwdCfg<256>::QB * 32 && kBQQ16 == kWaves * FwdCfg<128>::QB * 32,
              "query tile seen by the split plan");
#ifndef FA_FWDQ16_LA
#define FA_FWDQ16_LA 4
#endif
#ifndef FA_FWDQ16_128_WAVES
#define FA_FWDQ16_128_WAVES 4
#endif
// waves per SIMD the launch bounds ask the register allocation to allow: one
// workgroup (two waves per SIMD) per CU at d = 256, whose stages take 128 KB
// of LDS; two at d = 128 (64 KB each)
template <int D>
constexpr int q16_min_waves() { return D == 256 ? 2 : FA_FWDQ16_128_WAVES; }

// SPLITKV: the key tiles of each query tile are cut into a.splits ranges and
// each workgroup writes its range's O (fp32, normalised by its own sum) and
// LSE as partial rows, which fwd_merge_kernel combines (OUT_F32 unused).
template <int D, bool BF16, bool CAUSAL, bool OUT_F32, bool SPLITKV>
__global__ __launch_bounds__(kTQ16, q16_min_waves<D>()) void fwd_q16_kernel(FwdArgs a) {
  static_assert(D == 128 || D == 256, "the swizzles assume rows of one or two bank windows");
  constexpr int ROWB = D * 2;                     // bytes per K/V row
  constexpr int BK = kBKQ16, BQ = kBQQ16;
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  constexpr int DC = D / 32;                      // Q^T register groups (contraction of S^T)
  constexpr int DT = D / 16;                      // O^T accumulator tiles
  constexpr int LOADS = BK * CPR / kTQ16;         // direct loads per thread per tensor
  static_assert(LOADS * kTQ16 == BK * CPR, "tile split");
  constexpr int kTileLoads = 2 * LOADS;           // per thread per tile (K and V)
  constexpr int kAhead = kStQ16 - 1;              // prefetch distance in tiles
  constexpr int STAGEB = BK * ROWB;               // bytes per stage and tensor
  constexpr int LA = FA_FWDQ16_LA;

  __shared__ __attribute__((aligned(16))) uint16_t sK[kStQ16][BK * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kStQ16][BK * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15;  // this lane's query within the wave's 16 rows
  const int g = lane >> 4;  // its quarter of the wave

  int bh, qt, split = 0;
  {
    const int bid = blockIdx.x;
    const int S = SPLITKV ? a.splits : 1;
    if (CAUSAL) {
      qt = a.n_qtiles - 1 - bid / (a.BH * S);  // heaviest query tiles first
      const int rem = bid % (a.BH * S);
      bh = rem / S;
      split = rem % S;
    } else {
      // a head's query tiles on one XCD (ids are dealt round-robin over 8)
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
  const int qw0 = qt * BQ + wave * 16;  // first query row of this wave
  const int qrow = qw0 + m;

  // Q^T operand (B of S^T = K Q^T): register group dc holds d = 32dc + 8g ..
  // +7 of this lane's query row (rows past N read as 0).  Settled before the
  // loop, whose loads the compiler does not see.
  u32x4 qf[DC];
  {
    const brsrc_t rq = make_rsrc(a.q + base, head_bytes);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = bload16(rq, ((uint32_t)qrow * D + 32 * dc + 8 * g) * 2u, 0);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) settle(qf[dc]);
  }

  // K operand (A): key m of a 16-key block, chunk 4dc + g, stored at chunk
  // position (4dc + g) ^ (row & 15) (the XOR stays in the chunk's 256-byte
  // window, so offsets repeat every four dc).
  int kr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kr[i] = m * ROWB + (((4 * i + g) ^ m) * 16);
  auto k_off = [&](int dc) { return kr[dc & 3] + (dc >> 2) * 256; };
  // V^T operand (A of O^T += V^T P^T) through the transposing read: in
  // quarter g, lane 4j + q reads key 4g + j (16 + 4g + j for k-slots 4..7) at
  // d = 16dt + 4q .. +3, i.e. chunk 2dt + q/2 at position
  // (2dt + q/2) ^ 2(key & 7), bytes (q & 1) * 8; lane i then receives
  // d = 16dt + i for those four keys.
  // The V array starts 64 KB into LDS at d = 256, past what a read's 16-bit
  // offset field reaches, so each lane keeps its eight offsets with the
  // array's address already added (hidden from the compiler, which would
  // otherwise add the array's address back on every read); a read then adds
  // only the stage and window constants, which its offset field holds.
  uint32_t va[8];
  {
    const uint32_t lds_v0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&sV[0][0];
    const int j = m >> 2, q = m & 3, key = 4 * g + j;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      va[i] = lds_v0 + (uint32_t)(key * ROWB + (((2 * i + (q >> 1)) ^ ((key & 7) << 1)) * 16) + (q & 1) * 8);
      asm volatile("" : "+v"(va[i]));
    }
  }
  static_assert((kStQ16 - 1) * BK * ROWB + (D / 16 - 1) / 8 * 256 + 16 * ROWB + 8 < 65536,
                "V read constants fit the offset field");

  // Direct-load slots: thread slot p = i * kTQ16 + tid holds tile row p / CPR
  // at chunk position p % CPR, i.e. global chunk (p % CPR) ^ swz(row).
  uint32_t k_gl[LOADS], v_gl[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = i * kTQ16 + tid;
    const int row = p / CPR, pos = p % CPR;
    k_gl[i] = (uint32_t)(row * ROWB + ((pos ^ (row & 15)) * 16));
    v_gl[i] = (uint32_t)(row * ROWB + ((pos ^ ((row & 7) << 1)) * 16));
  }
  const u32x4 wk = rsrc_words(a.k + base, head_bytes);
  const u32x4 wv = rsrc_words(a.v + base, head_bytes);
  const uint32_t lds_k = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&sK[0][0];
  const uint32_t lds_v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&sV[0][0];
  const int kend = CAUSAL ? min(N, qt * BQ + BQ) : N;
  // This workgroup's key tiles: j0 .. j0 + n_kt - 1 (all of them unless split;
  // a split may hold none).
  int j0 = 0, n_kt = (kend + BK - 1) / BK;
  if constexpr (SPLITKV) {
    const int total = n_kt;
    j0 = (int)(((long long)split * total) / a.splits);
    n_kt = (int)(((long long)(split + 1) * total) / a.splits) - j0;
  }
  // local tile j (global tile j0 + j) into stage st
  auto issue_tile = [&](int j, int st) {
    const uint32_t soff =
        (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(j0 + j) * (uint32_t)STAGEB));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const uint32_t slot = (uint32_t)(st * STAGEB + (i * kTQ16 + wave * 64) * 16);
      bload16_lds_asm(wk, lds_k + slot, k_gl[i], soff);
      bload16_lds_asm(wv, lds_v + slot, v_gl[i], soff);
    }
  };

  const float c = a.c;

  // m_run: exponent reference (log2 units, the row's); l_run: this lane's
  // share of the sum of the rounded probabilities; l32_run: its fp32 sum (bf16
  // LSE).
  float m_run = -INFINITY, l_run = 0.f, l32_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // S^T of one K tile: s[kb][r] is key 16kb + 4g + r of the tile.
  struct S2 {
    f32x4 v[2];
  };
  auto scores = [&](const char* Kb) {
    S2 s;
    s.v[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    s.v[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4 ka = *(const u32x4*)(Kb + kb * 16 * ROWB + k_off(dc));
        s.v[kb] = mfma16<BF16>(ka, qf[dc], s.v[kb]);
        pin_step<1, 1, LA>(kb * DC + dc);
      }
    pin_tail<1, LA>();
    return s;
  };
  // O^T += V^T P^T for the packed probabilities pf (k-slot i: key
  // 4g + i for i < 4, 16 + 4g + i - 4 after).
  auto pv = [&](uint32_t vst, const u32x4& pf) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t at = va[dt & 7] + vst + (uint32_t)((dt >> 3) * 256);
      const u32x2 lo = lds_read_tr16_at(at);
      const u32x2 hi = lds_read_tr16_at(at + 16 * ROWB);
      const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
      oacc[dt] = mfma16<BF16>(vf, pf, oacc[dt]);
      pin_step<2, 2, LA>(dt);
    }
    pin_tail<2, LA>();
  };
  // p = 2^(c*s + neg_m) rounded to the input type and packed as the P^T
  // operand; ts: sum of the rounded values, ts32: their fp32 sum.
  auto exp_pack = [&](const S2& s, float neg_m, u32x4& pf, float& ts, float& ts32) {
    float p[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[4 * kb + r] = fast_exp2(__builtin_fmaf(s.v[kb][r], c, neg_m));
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pf[e] = pack2<BF16>(p[2 * e], p[2 * e + 1]);
      if (e & 1) t1 = sum2<BF16>(pf[e], t1); else t0 = sum2<BF16>(pf[e], t0);
    }
    ts = t0 + t1;
    if constexpr (BF16) ts32 = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  };
  auto row_max = [&](const S2& s) {
    const float a0 = fmaxf(fmaxf(s.v[0][0], s.v[0][1]), fmaxf(s.v[0][2], s.v[0][3]));
    const float a1 = fmaxf(fmaxf(s.v[1][0], s.v[1][1]), fmaxf(s.v[1][2], s.v[1][3]));
    return max4(fmaxf(a0, a1));
  };

  // Online softmax of one tile up to its packed probabilities.  MASK: the
  // causal diagonal and the end of the sequence.  The row max costs eight
  // compares and two exchanges here, so both types take it on every tile:
  // bf16 keeps the exact running max (the dominant probability is then
  // exactly 1), fp16 moves its reference only when the max rises more than 8
  // (log2 units) above it, which keeps every probability at most 2^8.  Rows
  // that do not move get alpha = 1 exactly.  The exponentials use the new
  // reference, so only the rescale of O (below) depends on whether a row
  // moved.
  auto softmax = [&](auto mask_tag, S2& s, int k0, u32x4& pf, float& alpha, bool& grow) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
      const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;  // last visible key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (k0 + 16 * kb + 4 * g + r > lim) s.v[kb][r] = -INFINITY;
    }
    const float mnew = row_max(s) * c;
    grow = mnew > m_run + rescale_threshold<BF16>();
    const float mn = grow ? mnew : m_run;
    alpha = grow ? ((m_run == -INFINITY) ? 0.f : fast_exp2(m_run - mn)) : 1.0f;
    m_run = mn;
    float ts, ts32 = 0.f;
    exp_pack(s, (mn == -INFINITY) ? 0.f : -mn, pf, ts, ts32);
    l_run = __builtin_fmaf(l_run, alpha, ts);
    if constexpr (BF16) l32_run = __builtin_fmaf(l32_run, alpha, ts32);
  };
  auto rescale_pv = [&](uint32_t vst, const u32x4& pf, float alpha, bool grow) {
    if (__ballot(grow) != 0ull) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    pv(vst, pf);
  };

  // Pipeline: iteration j (tile j in stage j % 4) starts tile j + 3's loads,
  // computes tile j + 1's scores alongside tile j's softmax (the MFMAs of the
  // one cover the exponentials of the other), then tile j's P V, and before
  // the barrier waits until tile j + 2 has landed: all but the newest tile's
  // loads (all of them once no load was started).  Past the last tile the
  // score read lands on a stage that is not being written and its result is
  // dropped.
  S2 s_cur;
  auto iteration = [&](int j, auto stage_tag) {
    constexpr int st = decltype(stage_tag)::value;
    constexpr int st1 = (st + 1) % kStQ16;
    if (j + kAhead < n_kt) issue_tile(j + kAhead, (st + kAhead) % kStQ16);
    const int k0 = (j0 + j) * BK;
    const bool active = !CAUSAL || (k0 <= qw0 + 15);
    if (active) {
      const bool need_mask = (k0 + BK > N) || (CAUSAL && k0 + BK - 1 > qw0);
      u32x4 pf;
      float alpha;
      bool grow;
      S2 s_next;
      if (need_mask) {
        s_next = scores((const char*)sK[st1]);
        softmax(std::true_type{}, s_cur, k0, pf, alpha, grow);
      } else {
        s_next = scores((const char*)sK[st1]);
        softmax(std::false_type{}, s_cur, k0, pf, alpha, grow);
      }
      rescale_pv((uint32_t)(st * STAGEB), pf, alpha, grow);
      s_cur = s_next;
    }
    if (j + kAhead < n_kt) {
      wait_vmem_keep<(kStQ16 - 3) * kTileLoads>();
    } else {
      wait_vmem();
    }
    barrier_no_fence();
  };

#pragma unroll
  for (int s0 = 0; s0 < kAhead; ++s0)
    if (s0 < n_kt) issue_tile(s0, s0);
  if (kAhead < n_kt) {
    wait_vmem_keep<(kStQ16 - 3) * kTileLoads>();  // tiles 0 and 1 have landed
  } else {
    wait_vmem();
  }
  barrier_no_fence();
  s_cur = scores((const char*)sK[0]);
  for (int j = 0; j < n_kt; j += kStQ16) {
    iteration(j, std::integral_constant<int, 0>{});
    if (j + 1 < n_kt) iteration(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 < n_kt) iteration(j + 2, std::integral_constant<int, 2>{});
    if (j + 3 < n_kt) iteration(j + 3, std::integral_constant<int, 3>{});
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
  // Lane (query m, quarter g) holds d = 16dt + 4g .. +3 of its row; rows past
  // N are dropped by the stores.
  if constexpr (SPLITKV) {
    // A row that saw no key in this range has l = 0: O = 0 and LSE = -inf,
    // which the merge weights by zero.  Partial rows r0 .. r0 + cnt - 1 of
    // the head.
    const int r0 = qt * BQ, cnt = min(BQ, N - r0);
    const size_t prow = (size_t)split * a.part_rows + (size_t)bh * N + r0 - a.part_row_base;
    const brsrc_t ro = make_rsrc(a.part_o + prow * D, (uint32_t)cnt * D * 4);
    const brsrc_t rl = make_rsrc(a.part_lse + prow, (uint32_t)cnt * 4);
    const int row = qrow - r0;
    const float lt = sum4(l_run);
    const float ll = BF16 ? sum4(l32_run) : lt;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = __float_as_uint(oacc[dt][t] * inv);
      bstore16(w, ro, ((uint32_t)row * D + (uint32_t)(16 * dt + 4 * g)) * 4u, 0);
    }
    if (g == 0) bstore4(ll > 0.f ? (m_run + fast_log2(ll)) * kLn2 : -INFINITY, rl, (uint32_t)row * 4u, 0);
    return;
  }
  const brsrc_t ro = make_rsrc((const char*)a.o + base * (OUT_F32 ? 4 : 2), (uint32_t)N * D * (OUT_F32 ? 4 : 2));
  const brsrc_t rl = make_rsrc(a.lse + (size_t)bh * N, (uint32_t)N * 4);
  const float lt = sum4(l_run);
  const float ll = BF16 ? sum4(l32_run) : lt;
  const float inv = 1.0f / lt;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const uint32_t col = (uint32_t)(16 * dt + 4 * g);
    if constexpr (OUT_F32) {
      u32x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = __float_as_uint(oacc[dt][t] * inv);
      bstore16(w, ro, ((uint32_t)qrow * D + col) * 4u, 0);
    } else {
      const u32x2 w = {pack2<BF16>(oacc[dt][0] * inv, oacc[dt][1] * inv),
                       pack2<BF16>(oacc[dt][2] * inv, oacc[dt][3] * inv)};
      bstore8(w, ro, ((uint32_t)qrow * D + col) * 2u, 0);
    }
  }
  if (g == 0) bstore4((m_run + fast_log2(ll)) * kLn2, rl, (uint32_t)qrow * 4u, 0);
}

template <int D, bool BF16, bool CAUSAL, bool OUT_F32, bool SPLITKV>
hipError_t launch_fwd_q16_t(const FwdProblem& p, hipStream_t stream) {
  FwdArgs a{};
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.o = p.o;
  a.lse = p.lse;
  a.N = p.N;
  a.BH = p.BH;
  a.n_qtiles = (p.N + kBQQ16 - 1) / kBQQ16;
  a.c = p.scale * kLog2e;
  a.splits = SPLITKV ? p.splits : 1;
  a.part_row_base = SPLITKV ? p.part_row_base : 0;
  a.part_rows = SPLITKV ? (p.part_rows > 0 ? p.part_rows : p.BH * p.N) : 0;
  a.part_o = SPLITKV ? p.part : nullptr;
  a.part_lse = SPLITKV ? p.part + (size_t)p.splits * a.part_rows * D : nullptr;
  a.item_base = CAUSAL ? 0 : p.item_base;
  const int n_items = p.item_count > 0 ? p.item_count : a.BH * a.n_qtiles - a.item_base;
  hipLaunchKernelGGL((fwd_q16_kernel<D, BF16, CAUSAL, SPLITKV ? false : OUT_F32, SPLITKV>),
                     dim3((unsigned)(n_items * a.splits)), dim3(kTQ16), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if constexpr (!SPLITKV) {
    return e;
  } else {
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
}

template <int D, bool SPLITKV>
hipError_t launch_fwd_q16(const FwdProblem& p, hipStream_t s) {
  const bool bf16 = p.dtype == kBF16 || p.dtype == kBF16OutF32;
  const bool f32 = p.dtype == kF16OutF32 || p.dtype == kBF16OutF32;
  if (p.dtype < kF16 || p.dtype > kBF16OutF32) return hipErrorInvalidValue;
  if (bf16) {
    if (f32)
      return p.causal ? launch_fwd_q16_t<D, true, true, true, SPLITKV>(p, s)
                      : launch_fwd_q16_t<D, true, false, true, SPLITKV>(p, s);
    return p.causal ? launch_fwd_q16_t<D, true, true, false, SPLITKV>(p, s)
                    : launch_fwd_q16_t<D, true, false, false, SPLITKV>(p, s);
  }
  if (f32)
    return p.causal ? launch_fwd_q16_t<D, false, true, true, SPLITKV>(p, s)
                    : launch_fwd_q16_t<D, false, false, true, SPLITKV>(p, s);
  return p.causal ? launch_fwd_q16_t<D, false, true, false, SPLITKV>(p, s)
                  : launch_fwd_q16_t<D, false, false, false, SPLITKV>(p, s);
}

}  // namespace fa
