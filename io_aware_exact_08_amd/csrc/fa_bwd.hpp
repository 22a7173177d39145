// Recompute-based backward of exact attention for gfx950.
//
// Page 2 of the subject, "Re-computation": no score or probability is kept
// from the forward; each (query tile, key tile) block recomputes
// S = scale Q K^T and P from it, with an outer loop over K/V column blocks and
// an inner loop over Q row blocks.  P is rebuilt with the forward's row LSE,
// P_ij = exp(scale q_i.k_j - LSE_i), which is the normalised softmax (the
// block-local softmax printed on that page would not be).  Gradients of
// L = <dO, O>:
//   D_i = sum_c dO_ic O_ic,  dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//   dK = scale dS^T Q,       dQ = scale dS K.
//
// Three kernels, all deterministic (no atomics):
//  * bwd_pre   : -D and -LSE*log2(e) for every row (one pass over O and dO).
//  * bwd_dkdv  : a workgroup keeps 128 keys of K and V in registers (32 per
//                wave) and loops over Q/dO tiles of 32 or 64 rows (dkdv_bq;
//                the loop order above); dK and dV accumulate in registers.
//  * bwd_dq    : a workgroup keeps 128 query rows of Q and dO in registers and
//                loops over K/V tiles of 32 or 64 keys (dq_bk).
// Mapping onto CDNA4, as in the forward: v_mfma_f32_32x32x16 with the
// accumulator of one product feeding the next as its B operand after
// rounding; streamed tiles arrive by direct buffer->LDS loads into two
// stages; operands that contract over tile rows are read with the
// transposing ds_read_b64_tr_b16 from the same row-major tile (one XOR
// swizzle serves both read patterns); the dP accumulator starts at -D so
// the MFMA produces dP - D; tiles on the causal diagonal run a masked copy of
// the tile body.  Rows and keys past N read as zeros and contribute nothing
// (their dO or K/V rows are zero), and stores past N are dropped.
#pragma once

#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr int kBwdThreads = 256;

// ---------------------------------------------------------------------------
// -D_i = -sum_c dO_ic O_ic and -LSE_i * log2(e)
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool O_F32>
__global__ __launch_bounds__(kBwdThreads) void bwd_pre_kernel(const void* __restrict__ o,
                                                              const uint16_t* __restrict__ dout,
                                                              const float* __restrict__ lse,
                                                              float* __restrict__ delta,
                                                              float* __restrict__ lse2, int rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  constexpr int RPB = kBwdThreads / LPR;
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / LPR;
  const int c = tid % LPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + c * 8;
    const u32x4 g = *(const u32x4*)(dout + off);
    float gv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gv[2 * e] = to_f32<BF16>((uint16_t)(g[e] & 0xffffu));
      gv[2 * e + 1] = to_f32<BF16>((uint16_t)(g[e] >> 16));
    }
    if constexpr (O_F32) {
      const f32x4 o0 = *(const f32x4*)((const float*)o + off);
      const f32x4 o1 = *(const f32x4*)((const float*)o + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += gv[e] * o0[e] + gv[4 + e] * o1[e];
    } else {
      const u32x4 ov = *(const u32x4*)((const uint16_t*)o + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += gv[2 * e] * to_f32<BF16>((uint16_t)(ov[e] & 0xffffu));
        acc += gv[2 * e + 1] * to_f32<BF16>((uint16_t)(ov[e] >> 16));
      }
    }
  }
#pragma unroll
  for (int w = 1; w < LPR; w <<= 1) acc += __shfl_xor(acc, w, 64);
  if (row < rows && c == 0) {
    // Both stored negated: they seed the dP - D and c*s - LSE*log2(e)
    // accumulators as they are.  A row whose every key is hidden (LSE = -inf,
    // O = 0) must recompute P = 0: its exponent reference is -inf.
    delta[row] = -acc;
    lse2[row] = lse[row] == -INFINITY ? -INFINITY : -(lse[row] * kLog2e);
  }
}

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse2;   // -LSE * log2(e)
  const float* delta;  // -D
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int N;
  int BH;
  int n_tiles;  // workgroup tiles per head
  float c;      // scale * log2(e)
  float scale;
  // additive attention bias (as in the forward), or null
  const uint16_t* bias;
  long long bias_sb, bias_sh;
  int H;
};

// Per-lane byte offsets shared by both kernels for a row-major LDS tile with
// ROWB bytes per row, swizzled with swz_dual (read both as a row operand and
// through the transposing read).
// The swizzles permute 16-byte chunks within one 256-byte bank window, so a
// lane's offsets repeat every window along a row (d=256 rows span two): only
// one window's worth is kept and the window offset is added as an immediate.
template <int D>
struct TileOffsets {
  static constexpr int ROWB = D * 2;
  static constexpr int DC = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int RDC = DC < 8 ? DC : 8;
  static constexpr int RDT = DT < 4 ? DT : 4;
  int rd_[RDC];   // row operand: rows 32t + perm_k(m), chunk 2dc+h (+ 32t*ROWB)
  int trl_[RDT];  // transposing read for d tile dt, k-rows 8h + j (+ 16kc*ROWB)
  int trh_[RDT];  // the same for k-rows 8h + 4 + j
  __device__ __forceinline__ int rd(int dc) const { return rd_[dc % RDC] + (dc / RDC) * 256; }
  __device__ __forceinline__ int trl(int dt) const { return trl_[dt % RDT] + (dt / RDT) * 256; }
  __device__ __forceinline__ int trh(int dt) const { return trh_[dt % RDT] + (dt / RDT) * 256; }
  __device__ __forceinline__ TileOffsets(int lane) {
    const int m = lane & 31, h = lane >> 5;
    const int row = perm_k(m);
#pragma unroll
    for (int dc = 0; dc < RDC; ++dc) rd_[dc] = row * ROWB + (((2 * dc + h) ^ swz_dual<D>(row)) * 16);
    const int i = lane & 15, gg = (lane >> 4) & 1;
    const int j = i >> 2, q = i & 3;
    const int trow = 8 * h + j;
#pragma unroll
    for (int dt = 0; dt < RDT; ++dt) {
      const int chunk = 4 * dt + 2 * (q & 1) + gg;
      trl_[dt] = trow * ROWB + ((chunk ^ swz_dual<D>(trow)) * 16) + (q >> 1) * 8;
      trh_[dt] = (trow + 4) * ROWB + ((chunk ^ swz_dual<D>(trow + 4)) * 16) + (q >> 1) * 8;
    }
  }
};

// Direct-load slot p = i*256 + tid of a tile of rows x CPR 16-byte chunks:
// tile row p / CPR at swizzled chunk position p % CPR.
template <int D>
__device__ __forceinline__ uint32_t tile_src_offset(int p) {
  constexpr int CPR = D / 8;
  const int row = p / CPR, cpos = p % CPR;
  return (uint32_t)(row * D * 2 + ((cpos ^ swz_dual<D>(row)) * 16));
}

// Transposed operand (A of an O^T-shaped product) for 16 k-rows starting at
// tile row 16*kc from the transposing reads.
__device__ __forceinline__ u32x4 tr_operand(const char* tile, int off_lo, int off_hi, int kc,
                                            int rowb) {
  const u32x2 lo = lds_read_tr16(tile + off_lo + kc * 16 * rowb);
  const u32x2 hi = lds_read_tr16(tile + off_hi + kc * 16 * rowb);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

template <int D>
constexpr int bwd_min_waves() { return D == 64 ? 2 : 1; }

// Operand reads issued this many MFMAs ahead of their MFMA (pin_step).  Left
// to itself the scheduler hoists a tile's transposing reads far ahead: the
// causal dK/dV instantiations reached 320 live registers before allocation
// and spilled 16.  Measured on MI355X, lookahead 4 against none: causal
// dK/dV -23% (N=4096) and -20% (N=32768), non-causal dK/dV -1%, dQ -1.5%
// (non-causal) to -7% (causal N=4096); lookahead 2, 6 and 8 were slower.
// With the log2-unit scores (fewer VALU instructions per tile) lookahead 3
// beat 4 on every backward shape measured: dK/dV -0.8% (B2 H12 N8192 fp16),
// -2.4% (causal N=4096), -0.9% (B1 H8 N32768 bf16 causal), dQ -0.4 to -1.1%;
// 5 and 6 were not faster than 4.
#ifndef FA_BWD_PIN_LA
#define FA_BWD_PIN_LA 3
#endif
// Order of the second product chain (dV/dK, dQ): contraction chunk outermost,
// so its first half needs only the first 32-row half of P and dS and the
// second half's exponentials can run under those MFMAs.  Measured on MI355X
// against d-tile outermost: causal dK/dV -1.7% (B2 H12 N4096 fp16), dQ -1.5%
// (B1 H8 N32768 bf16 causal) and -0.5% (B2 H12 N8192 fp16), others unchanged.
// Hand-counted direct loads for the unbiased kernels (the bias kernels always
// count theirs).  Same-box A/B against the compiler's waits: d=128 non-causal
// dQ -9.8% and dK/dV -1.1% (B2 H12 N4096 fp16), so those use them; at d=64
// the headline shape moved within +-1.5%, causal N=4096 dQ +2.6%, B1 H8
// N32768 bf16 causal dQ -2.9%, d=128 bf16 causal dQ +1.9%, dK/dV -2.1%.
// d=256 (one wave per SIMD): counted loads measured dQ -7% (B2 H8 N4096
// fp16), -6.5% (bf16), -11% (bf16 causal); dK/dV within 0.5%, -2.2% causal.
#ifndef FA_BWD256_COUNTED
#define FA_BWD256_COUNTED 1
#endif
#ifndef FA_BWD_COUNTED
#define FA_BWD_COUNTED 0
#endif
#ifndef FA_BWD_PRESCALE
#define FA_BWD_PRESCALE 1
#endif
#ifndef FA_BWD_CHUNK_MAJOR
#define FA_BWD_CHUNK_MAJOR 1
#endif

// ---------------------------------------------------------------------------
// dK, dV: workgroup owns 128 keys (32 per wave); loop over query tiles.
// ---------------------------------------------------------------------------
constexpr int kDkvKeys = 128;  // keys per workgroup
constexpr int kDkvBQ = 64;     // query rows per streamed tile, unless 32 below
// d=256 streams 32-row tiles: its K/V fragments take 128 registers per lane
// and its dK/dV accumulators 256 (in the accumulation registers), which
// leaves room for one 32-row tile's scores and dP only.
// d=128 (unbiased, except fp16 causal) streams 32-row tiles as well: the
// smaller score and dP tiles let the non-causal kernels run two waves per
// SIMD with nothing parked in the accumulation registers (B2 H12 N4096:
// -11% fp16, -14% bf16; bf16 causal -4%; fp16 causal measured +3% and keeps
// 64 rows, as do the bias kernels).  So does the unbiased non-causal d=64
// one, which then runs three waves per SIMD (165 VGPRs): -6% at B2 H12
// N4096, -1% at N8192; its causal kernels measured 6-16% slower.
template <int D, bool BF16, bool CAUSAL, bool BIAS>
__host__ __device__ constexpr int dkdv_bq() {
  return D == 256 ? 32
       : (D == 128 && !BIAS && !(CAUSAL && !BF16)) ? 32
       : (D == 64 && !BIAS && !CAUSAL)              ? 32
                                                    : kDkvBQ;
}

template <int D, int BQ>
__host__ __device__ constexpr int dkdv_stage_bytes() {
  return 2 * BQ * D * 2 + 2 * BQ * 4;  // Q, dO tiles + LSE2, D rows
}

template <int D, bool BF16, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kBwdThreads, bwd_min_waves<D>()) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BQ = dkdv_bq<D, BF16, CAUSAL, BIAS>();
  constexpr int DC = D / 16;
  constexpr int DT = D / 32;
  constexpr int QT = BQ / 32;  // 32-row query sub-tiles per streamed tile
  constexpr int QC = BQ / 16;  // 16-row query chunks (contraction of dK, dV)
  constexpr int CPR = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int LOADS = BQ * CPR / kBwdThreads;
  static_assert(LOADS * kBwdThreads == BQ * CPR, "tile split");
  // With a bias every direct load of the query loop is issued as inline
  // assembly and waited for by hand, and each wave stages its 32 key columns
  // of the bias two query tiles ahead in an LDS ring behind the two stages
  // (see the forward: the compiler would otherwise wait for all direct loads
  // before each LDS read).
  constexpr bool kCounted = BIAS || FA_BWD_COUNTED || (D == 128 && !CAUSAL) || (D == 256 && FA_BWD256_COUNTED);
  constexpr bool kBiasLds = BIAS;
  constexpr int STAGE = dkdv_stage_bytes<D, BQ>();
  constexpr int TILE = BQ * ROWB;
  // fp16: K is pre-multiplied by c = scale*log2(e) and the S accumulators
  // start at -LSE*log2(e) (as dP's start at -D), so the MFMAs produce the
  // exponent c*s - LSE*log2(e) itself: no multiply-add per score (a bias then
  // adds bias*log2(e), and a zero bias changes nothing).  bf16 keeps the
  // scale in fp32: rounding K*c to 8 bits tripled the gradient error at
  // scale 1 (1.6e-2 against 5e-3; fp16: 2e-3).
  // (d=256 keeps the scale in fp32 too: seeding S from LDS keeps 16 more
  // registers live, and its non-causal fp16 kernel then spilled 33)
  constexpr bool PRE = FA_BWD_PRESCALE && !BF16 && D != 256;

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 31, h = lane >> 5;

  int bh, kvt;
  {
    const int bid = blockIdx.x;
    if (CAUSAL) {
      kvt = bid / a.BH;  // first key tiles see the most queries: issue first
      bh = bid % a.BH;
    } else {
      const int G = gridDim.x;
      const int lin = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
      bh = lin / a.n_tiles;
      kvt = lin % a.n_tiles;
    }
  }
  const int N = a.N;
  const size_t base = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const brsrc_t rq = make_rsrc(a.q + base, head_bytes);
  const brsrc_t rg = make_rsrc(a.dout + base, head_bytes);
  const brsrc_t rl = make_rsrc(a.lse2 + (size_t)bh * N, (uint32_t)N * 4);
  const brsrc_t rd = make_rsrc(a.delta + (size_t)bh * N, (uint32_t)N * 4);
  const int kw0 = kvt * kDkvKeys + wave * 32;  // first key of this wave
  const int key = kw0 + m;                     // this lane's key (column of S)
  // Bias gather through the transposing read from the bias ring, whose rows
  // are this wave's 32 keys (64 bytes): in each 16-lane group (G), lane L
  // supplies row R + L/4 and columns 16(G%2) + 4(L%4) .. +3; result lane i
  // then holds rows R..R+3 of column 16(G%2) + i.  With R = 32t + 16g +
  // 8(G/2) (+4), lane l receives exactly the bias of its key (l%32) at the
  // query rows of score registers 8g + 0..3 (and 4..7) of sub-tile t.  Four
  // rows fill a 256-byte bank window, so the 32 lanes of a read cycle (rows
  // R..R+3, both column halves) hit every bank slot once.
  constexpr int kRingRowBytes = 64;
  const int bias_rd_w = ((lane & 15) >> 2) * kRingRowBytes + 8 * ((lane >> 5) & 1) * kRingRowBytes +
                        (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  // K and V as B operands (lane: key m; slot i: d = 16dc + 8h + i).
  u32x4 kf[DC], vf[DC];
  {
    const brsrc_t rk = make_rsrc(a.k + base, head_bytes);
    const brsrc_t rv = make_rsrc(a.v + base, head_bytes);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const uint32_t off = ((uint32_t)key * D + dc * 16 + 8 * h) * 2u;
      kf[dc] = bload16(rk, off, 0);
      vf[dc] = bload16(rv, off, 0);
    }
    if constexpr (PRE) {
      // K * c rounded to the input type once: the S MFMAs then yield c*s
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = kf[dc][e];
          kf[dc][e] = pack2<BF16>(to_f32<BF16>((uint16_t)(w & 0xffffu)) * a.c,
                                  to_f32<BF16>((uint16_t)(w >> 16)) * a.c);
        }
    }
    if constexpr (kCounted) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        settle(kf[dc]);
        settle(vf[dc]);
      }
    }
  }
  const TileOffsets<D> to(lane);
  uint32_t src[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) src[i] = tile_src_offset<D>(i * kBwdThreads + tid);

  f32x16 dkt[DT], dvt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dkt[dt] = f32x16{};
    dvt[dt] = f32x16{};
  }

  const int n_qt = (N + BQ - 1) / BQ;
  const int qt_begin = CAUSAL ? (kvt * kDkvKeys) / BQ : 0;

  // hand-counted loads (bias only): resource words and 32-bit LDS addresses
  u32x4 wq{}, wg{}, wl{}, wb{};
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)smem;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (kCounted) {
    wq = rsrc_words(a.q + base, head_bytes);
    wg = rsrc_words(a.dout + base, head_bytes);
    // waves 0, 1 load the LSE2 row, waves 2, 3 the D row (a quarter each)
    wl = wave_u < 2 ? rsrc_words(a.lse2 + (size_t)bh * N, (uint32_t)N * 4)
                    : rsrc_words(a.delta + (size_t)bh * N, (uint32_t)N * 4);
  }
  if constexpr (kBiasLds)
    wb = rsrc_words(a.bias + (bh / a.H) * a.bias_sb + (bh % a.H) * a.bias_sh, (uint32_t)N * N * 2);
  // `live` false: a tile past the end, read from past the resource (nothing
  // moves), so that the loads in flight keep a fixed pattern.
  auto issue_tile_counted = [&](int qt, char* stage, bool live) {
    const uint32_t st = lds0 + (uint32_t)(stage - smem);
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(live ? (uint32_t)qt * (uint32_t)(BQ * ROWB) : head_bytes));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const uint32_t slot = (uint32_t)((i * kBwdThreads + wave_u * 64) * 16);
      bload16_lds_asm(wq, st + slot, src[i], soff);
      bload16_lds_asm(wg, st + TILE + slot, src[i], soff);
    }
    // the BQ LSE2 and BQ D values (2 * BQ * 4 bytes): one load per wave, by
    // its first BQ / 8 lanes only (a direct load writes every active lane's
    // slot, zeros past the resource included)
    const uint32_t lsoff = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(live ? (uint32_t)qt * (uint32_t)(BQ * 4) : (uint32_t)N * 4u));
    const uint32_t part = (uint32_t)((wave_u & 1) * (BQ * 2));  // byte offset within the row slice
    if (lane < BQ / 8)
      bload16_lds_asm(wl, st + 2 * TILE + (wave_u >> 1) * (BQ * 4) + part, part + (uint32_t)(lane * 16), lsoff);
  };
  auto issue_tile = [&](int qt, char* stage) {
    const uint32_t soff = (uint32_t)qt * (uint32_t)(BQ * ROWB);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = (i * kBwdThreads + wave * 64) * 16;
      bload16_lds(rq, stage + slot, src[i], soff);
      bload16_lds(rg, stage + TILE + slot, src[i], soff);
    }
    // BQ LSE2 and BQ D values: BQ/4 lanes of waves 0 and 1.
    if (lane < BQ / 4) {
      if (wave == 0) bload16_lds(rl, stage + 2 * TILE, (uint32_t)(lane * 16), (uint32_t)qt * (uint32_t)(BQ * 4));
      if (wave == 1) bload16_lds(rd, stage + 2 * TILE + BQ * 4, (uint32_t)(lane * 16), (uint32_t)qt * (uint32_t)(BQ * 4));
    }
  };

  // Bias ring: wave w, slot t % 2 holds rows t*BQ .. +63 of its 32 keys
  // (64 bytes a row); direct load i, lane l fills bytes 16(64i + l), i.e. row
  // (64i + l) / 4, 16-byte chunk l % 4.  Tile t's bias follows tile t - 1's
  // Q/dO in issue order (as the loop below issues them), so when it is read
  // the Q/dO of tiles t and t + 1 and tile t + 1's bias are newer; at the
  // end of iteration t only tile t + 2's bias is newer than tile t + 1's Q/dO.
  constexpr int LB = BQ * kRingRowBytes / 16 / 64;  // direct loads per lane per tile
  constexpr int kTileLoads = 2 * LOADS + 1;
  const int ring_off = 2 * STAGE;
  uint32_t b_gl[kBiasLds ? LB : 1];
  if constexpr (kBiasLds) {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int p = i * 64 + lane;
      b_gl[i] = ((uint32_t)(p / 4) * (uint32_t)N + (uint32_t)(kw0 + (p % 4) * 8)) * 2u;
    }
  }
  auto issue_bias = [&](int t, bool live) {
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(live ? (uint32_t)t * (uint32_t)BQ * (uint32_t)N * 2u : (uint32_t)N * (uint32_t)N * 2u));
    const uint32_t slot = lds0 + (uint32_t)(ring_off + (wave_u * 2 + (t & 1)) * BQ * kRingRowBytes);
#pragma unroll
    for (int i = 0; i < LB; ++i) bload16_lds_asm(wb, slot + i * 64 * 16, b_gl[i], soff);
  };

  const float c = a.c;
  // `after_bias`: called once the tile's bias has been read (bias ring only)
  auto tile_body = [&](auto mask_tag, const char* stage, int q0, auto&& after_bias) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* sQ = stage;
    const char* sG = stage + TILE;
    const float* sL = (const float*)(stage + 2 * TILE);
    const float* sD = sL + BQ;
    // S = Q K^T; dP - D = dO V^T - D (rows: queries with perm_k, cols: keys).
    // Register r of sub-tile t holds query row t*32 + 16(r/8) + 8h + r%8.
    f32x16 s[QT], dp[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      s[t] = f32x16{};
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int qb = t * 32 + 16 * g + 8 * h;
        const f32x4 d0 = *(const f32x4*)(&sD[qb]);
        const f32x4 d1 = *(const f32x4*)(&sD[qb + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dp[t][8 * g + e] = d0[e];
          dp[t][8 * g + 4 + e] = d1[e];
        }
        if constexpr (PRE) {
          const f32x4 l0 = *(const f32x4*)(&sL[qb]);
          const f32x4 l1 = *(const f32x4*)(&sL[qb + 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[t][8 * g + e] = l0[e];
            s[t][8 * g + 4 + e] = l1[e];
          }
        }
      }
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4 qa = *(const u32x4*)(sQ + t * 32 * ROWB + to.rd(dc));
        const u32x4 ga = *(const u32x4*)(sG + t * 32 * ROWB + to.rd(dc));
        s[t] = mfma32<BF16>(qa, kf[dc], s[t]);
        pin_step<1, 1, FA_BWD_PIN_LA>(2 * (t * DC + dc));
        dp[t] = mfma32<BF16>(ga, vf[dc], dp[t]);
        pin_step<1, 1, FA_BWD_PIN_LA>(2 * (t * DC + dc) + 1);
      }
    }
    pin_tail<1, FA_BWD_PIN_LA>();
    if constexpr (BIAS) {
      // s + bias/scale (so that c * s = scale*q.k*log2(e) + bias*log2(e));
      // with PRE the scores are already in log2 units: s + bias*log2(e)
      const float kb = PRE ? kLog2e : 1.0f / a.scale;
      const char* sB = smem + ring_off + (wave * 2 + ((q0 / BQ) & 1)) * BQ * kRingRowBytes;
      u32x2 bv[QT][2][2];
      wait_vmem_keep<2 * kTileLoads + LB>();  // this tile's bias has landed
#pragma unroll
      for (int t = 0; t < QT; ++t)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int half = 0; half < 2; ++half)
            bv[t][g][half] = lds_read_tr16(sB + bias_rd_w + (t * 32 + 16 * g + 4 * half) * kRingRowBytes);
      after_bias();
#pragma unroll
      for (int t = 0; t < QT; ++t)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const u32x2 w = bv[t][g][half];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 8 * g + 4 * half + 2 * e;
              s[t][r] = __builtin_fmaf(to_f32<BF16>((uint16_t)(w[e] & 0xffffu)), kb, s[t][r]);
              s[t][r + 1] = __builtin_fmaf(to_f32<BF16>((uint16_t)(w[e] >> 16)), kb, s[t][r + 1]);
            }
          }
    }
    u32x4 pp[QC], ps[QC];
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int qb = t * 32 + 16 * g + 8 * h;
        const f32x4 l0 = *(const f32x4*)(&sL[qb]);  // -LSE*log2(e) (unused with PRE)
        const f32x4 l1 = *(const f32x4*)(&sL[qb + 4]);
        float pv[8], dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float p;
          if constexpr (PRE) {
            p = fast_exp2(s[t][8 * g + e]);
          } else {
            const float nl2 = e < 4 ? l0[e] : l1[e - 4];
            p = fast_exp2(__builtin_fmaf(s[t][8 * g + e], c, nl2));
          }
          if constexpr (MASK) {
            if (key > q0 + qb + e) p = 0.f;
          }
          pv[e] = p;
          dsv[e] = p * dp[t][8 * g + e];
        }
        u32x4 wp, wd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wp[e] = pack2<BF16>(pv[2 * e], pv[2 * e + 1]);
          wd[e] = pack2<BF16>(dsv[2 * e], dsv[2 * e + 1]);
        }
        pp[2 * t + g] = wp;
        ps[2 * t + g] = wd;
      }
    // dV^T += dO^T P ; dK^T += Q^T dS   (rows: d with perm_o, cols: keys)
#pragma unroll
    for (int i = 0; i < DT * QC; ++i) {
      const int dt = FA_BWD_CHUNK_MAJOR ? i % DT : i / QC;
      const int qc = FA_BWD_CHUNK_MAJOR ? i / DT : i % QC;
      const u32x4 ga = tr_operand(sG, to.trl(dt), to.trh(dt), qc, ROWB);
      const u32x4 qa = tr_operand(sQ, to.trl(dt), to.trh(dt), qc, ROWB);
      dvt[dt] = mfma32<BF16>(ga, pp[qc], dvt[dt]);
      pin_step<2, 2, FA_BWD_PIN_LA>(2 * i);
      dkt[dt] = mfma32<BF16>(qa, ps[qc], dkt[dt]);
      pin_step<2, 2, FA_BWD_PIN_LA>(2 * i + 1);
    }
    pin_tail<2, FA_BWD_PIN_LA>();
  };

  auto iteration = [&](int qt, char* cur, char* nxt) {
    if constexpr (kBiasLds) {
      issue_tile_counted(qt + 1, nxt, qt + 1 < n_qt);
    } else if constexpr (kCounted) {
      if (qt + 1 < n_qt) issue_tile_counted(qt + 1, nxt, true);
    } else {
      if (qt + 1 < n_qt) issue_tile(qt + 1, nxt);
    }
    const int q0 = qt * BQ;
    const bool active = !CAUSAL || (q0 + BQ - 1 >= kw0);
    // the ring slot of tile qt is refilled with tile qt + 2's bias as soon as
    // it has been read (on a skipped tile: right away)
    auto refill = [&]() {
      if constexpr (kBiasLds) {
        wait_lds();
        issue_bias(qt + 2, qt + 2 < n_qt);
      }
    };
    if (active) {
      // d=256: keep each tile's body in its own scheduling region (overlapped
      // with the next one the non-causal kernel spilled ~190 registers)
      if constexpr (D == 256) __builtin_amdgcn_sched_barrier(0);
      if (CAUSAL && q0 < kw0 + 31) {
        tile_body(std::true_type{}, cur, q0, refill);
      } else {
        tile_body(std::false_type{}, cur, q0, refill);
      }
      if constexpr (D == 256) __builtin_amdgcn_sched_barrier(0);
    } else {
      refill();
    }
    if constexpr (kBiasLds) {
      wait_vmem_keep<LB>();
      barrier_no_fence();
    } else if constexpr (kCounted) {
      wait_vmem();
      barrier_no_fence();
    } else {
      wait_vmem();
      __syncthreads();
    }
  };

  char* st0 = smem;
  char* st1 = smem + STAGE;
  if constexpr (kCounted && !kBiasLds) {
    if (qt_begin < n_qt) issue_tile_counted(qt_begin, st0, true);
    wait_vmem();
    barrier_no_fence();
  } else if constexpr (kBiasLds) {
    issue_bias(qt_begin, qt_begin < n_qt);
    issue_tile_counted(qt_begin, st0, qt_begin < n_qt);
    issue_bias(qt_begin + 1, qt_begin + 1 < n_qt);
    wait_vmem_keep<LB>();  // tile qt_begin's Q/dO (and so its bias)
    barrier_no_fence();
  } else {
    if (qt_begin < n_qt) issue_tile(qt_begin, st0);
    wait_vmem();
    __syncthreads();
  }
  if constexpr (D == 256) {
    // one tile body per loop trip, stages swapped at run time (unrolled by
    // two, the non-causal kernel spilled ~190 registers)
    for (int qt = qt_begin; qt < n_qt; ++qt) {
      iteration(qt, st0, st1);
      char* t = st0;
      st0 = st1;
      st1 = t;
    }
  } else {
    for (int qt = qt_begin; qt < n_qt; qt += 2) {
      iteration(qt, st0, st1);
      if (qt + 1 < n_qt) iteration(qt + 1, st1, st0);
    }
  }
  if constexpr (kBiasLds) wait_vmem();  // (the ring's loads past the end)

  // dK = scale dS^T Q, dV: lane (key m, half h) holds d = 32dt + 16h + r.
  const brsrc_t rdk = make_rsrc(a.dk + base, head_bytes);
  const brsrc_t rdv = make_rsrc(a.dv + base, head_bytes);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const uint32_t off = ((uint32_t)key * D + dt * 32 + 16 * h) * 2u;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      u32x4 wk, wv;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        wk[t] = pack2<BF16>(dkt[dt][8 * e + 2 * t] * a.scale, dkt[dt][8 * e + 2 * t + 1] * a.scale);
        wv[t] = pack2<BF16>(dvt[dt][8 * e + 2 * t], dvt[dt][8 * e + 2 * t + 1]);
      }
      bstore16(wk, rdk, off + 16 * e, 0);
      bstore16(wv, rdv, off + 16 * e, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup owns 128 query rows (32 per wave); loop over key tiles.
// ---------------------------------------------------------------------------
constexpr int kDqRows = 128;
// keys per streamed K/V tile (d=256: 32, for the same register reason as the
// dK/dV kernel's 32-row tiles)
// (unbiased d=128 streams 32-key tiles too: -2% to -7%, the causal kernels
// then running two waves per SIMD; bf16 non-causal +1.4%)
template <int D, bool BIAS>
__host__ __device__ constexpr int dq_bk() { return D == 256 ? 32 : (D == 128 && !BIAS) ? 32 : 64; }

template <int D, bool BIAS>
__host__ __device__ constexpr int dq_stage_bytes() {
  return 2 * dq_bk<D, BIAS>() * D * 2;  // K, V tiles
}
// With a bias each wave stages its 32 rows of two key tiles' bias in LDS
// (see bwd_dq_kernel), behind the two K/V stages.
template <int D, bool BIAS>
__host__ __device__ constexpr int dq_ring_bytes() {
  return BIAS ? (kBwdThreads / 64) * 2 * 32 * dq_bk<D, BIAS>() * 2 : 0;
}

template <int D, bool BF16, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kBwdThreads, bwd_min_waves<D>()) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BK = dq_bk<D, BIAS>();
  constexpr int DC = D / 16;
  constexpr int DT = D / 32;
  constexpr int KT = BK / 32;
  constexpr int KC = BK / 16;
  constexpr int CPR = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int LOADS = BK * CPR / kBwdThreads;
  static_assert(LOADS * kBwdThreads == BK * CPR, "tile split");
  constexpr int STAGE = dq_stage_bytes<D, BIAS>();
  constexpr int TILE = BK * ROWB;
  // fp16: Q is pre-multiplied by c and the S accumulators start at
  // -LSE*log2(e) (this lane's row), as in the dK/dV kernel.
  constexpr bool PRE = FA_BWD_PRESCALE && !BF16;
  // With a bias every direct load of the key loop is issued as inline
  // assembly and waited for by hand, and each wave stages its bias rows two
  // key tiles ahead in an LDS ring (the forward's scheme: the compiler would
  // otherwise wait for all direct loads before each LDS read).
  constexpr bool kCounted = BIAS || FA_BWD_COUNTED || (D == 128 && !CAUSAL) || (D == 256 && FA_BWD256_COUNTED);
  constexpr bool kBiasLds = BIAS;

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 31, h = lane >> 5;

  int bh, qt;
  {
    const int bid = blockIdx.x;
    if (CAUSAL) {
      qt = a.n_tiles - 1 - bid / a.BH;
      bh = bid % a.BH;
    } else {
      const int G = gridDim.x;
      const int lin = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
      bh = lin / a.n_tiles;
      qt = lin % a.n_tiles;
    }
  }
  const int N = a.N;
  const size_t base = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const brsrc_t rk = make_rsrc(a.k + base, head_bytes);
  const brsrc_t rv = make_rsrc(a.v + base, head_bytes);
  const int qw0 = qt * kDqRows + wave * 32;
  const int qrow = qw0 + m;

  // Q^T and dO^T as B operands (lane: query m; slot i: d = 16dc + 8h + i).
  u32x4 qf[DC], gf[DC];
  {
    const brsrc_t rq = make_rsrc(a.q + base, head_bytes);
    const brsrc_t rg = make_rsrc(a.dout + base, head_bytes);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const uint32_t off = ((uint32_t)qrow * D + dc * 16 + 8 * h) * 2u;
      qf[dc] = bload16(rq, off, 0);
      gf[dc] = bload16(rg, off, 0);
    }
    if constexpr (PRE) {
      // Q * c rounded to the input type once: the S MFMAs then yield c*s
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = qf[dc][e];
          qf[dc][e] = pack2<BF16>(to_f32<BF16>((uint16_t)(w & 0xffffu)) * a.c,
                                  to_f32<BF16>((uint16_t)(w >> 16)) * a.c);
        }
    }
  }
  // Rows past N: LSE2 and D read as 0; their Q and dO rows are 0 and dQ is
  // not stored.
  float nl2, dl;  // -LSE * log2(e) and -D of this lane's query row
  {
    const brsrc_t rl = make_rsrc(a.lse2 + (size_t)bh * N, (uint32_t)N * 4);
    const brsrc_t rd = make_rsrc(a.delta + (size_t)bh * N, (uint32_t)N * 4);
    nl2 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, qrow * 4, 0, 0));
    dl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, qrow * 4, 0, 0));
  }
  if constexpr (kCounted) {
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      settle(qf[dc]);
      settle(gf[dc]);
    }
    settle(nl2);
    settle(dl);
  }
  const TileOffsets<D> to(lane);
  uint32_t src[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) src[i] = tile_src_offset<D>(i * kBwdThreads + tid);

  f32x16 dqt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqt[dt] = f32x16{};

  const int kend = CAUSAL ? min(N, qt * kDqRows + kDqRows) : N;
  const int n_kt = (kend + BK - 1) / BK;

  // hand-counted loads (bias only): resource words and 32-bit LDS addresses
  u32x4 wk{}, wv{}, wb{};
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)smem;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (kCounted) {
    wk = rsrc_words(a.k + base, head_bytes);
    wv = rsrc_words(a.v + base, head_bytes);
  }
  if constexpr (kBiasLds)
    wb = rsrc_words(a.bias + (bh / a.H) * a.bias_sb + (bh % a.H) * a.bias_sh, (uint32_t)N * N * 2);
  // `live` false: a tile past the end, read from past the resource (nothing
  // moves), so that the loads in flight keep a fixed pattern.
  auto issue_tile = [&](int j, char* stage, bool live = true) {
    if constexpr (kCounted) {
      const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(live ? (uint32_t)j * (uint32_t)(BK * ROWB) : head_bytes));
      const uint32_t st = lds0 + (uint32_t)(stage - smem);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t slot = (uint32_t)((i * kBwdThreads + wave_u * 64) * 16);
        bload16_lds_asm(wk, st + slot, src[i], soff);
        bload16_lds_asm(wv, st + TILE + slot, src[i], soff);
      }
    } else {
      const uint32_t soff = (uint32_t)j * (uint32_t)(BK * ROWB);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int slot = (i * kBwdThreads + wave * 64) * 16;
        bload16_lds(rk, stage + slot, src[i], soff);
        bload16_lds(rv, stage + TILE + slot, src[i], soff);
      }
    }
  };

  // Bias ring (the forward's layout): wave w, slot t % 2 holds its 32 rows x
  // BK keys of tile t, row-major, 16-byte chunk c of row r at position
  // c ^ swz_b(r); direct load i, lane l fills slot position 64i + l.
  constexpr int CPRB = BK / 8;
  constexpr int RPW = 256 / (BK * 2);
  constexpr int LB = 32 * CPRB / 64;  // direct loads per lane per tile
  auto swz_b = [](int row) { return (row / RPW) % CPRB; };
  const int ring_off = 2 * STAGE;
  uint32_t b_gl[kBiasLds ? LB : 1];
  if constexpr (kBiasLds) {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int p = i * 64 + lane;
      const int row = p / CPRB, pos = p % CPRB;
      b_gl[i] = (uint32_t)(qw0 + row) * (uint32_t)N * 2u + (uint32_t)((pos ^ swz_b(row)) * 16);
    }
  }
  auto issue_bias = [&](int t, bool live) {
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(live ? (uint32_t)t * (uint32_t)(BK * 2) : (uint32_t)N * (uint32_t)N * 2u));
    const uint32_t slot = lds0 + (uint32_t)(ring_off + (wave_u * 2 + (t & 1)) * 32 * BK * 2);
#pragma unroll
    for (int i = 0; i < LB; ++i) bload16_lds_asm(wb, slot + i * 64 * 16, b_gl[i], soff);
  };

  const float c = a.c;
  // this lane's bias for keys 32kt + 16g + 8h + 0..7 of a tile, read from the
  // ring
  auto read_bias = [&](int j, u32x4 (&bw)[KT][2]) {
    const char* bb = smem + ring_off + (wave * 2 + (j & 1)) * 32 * BK * 2;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        bw[kt][g] = *(const u32x4*)(bb + m * (BK * 2) + (((4 * kt + 2 * g + h) ^ swz_b(m)) * 16));
  };
  auto tile_body = [&](auto mask_tag, const char* stage, int k0, const u32x4 (&bw_ring)[KT][2]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* sK = stage;
    const char* sV = stage + TILE;
    // S^T = K Q^T, dP^T - D = V dO^T - D (rows: keys with perm_k, cols:
    // queries).  Register r of key tile kt holds key kt*32 + 16(r/8) + 8h + r%8.
    // With a bias, registers 8g..8g+7 of key tile kt take eight consecutive
    // entries of this lane's bias row, read from the ring before the tile.
    u32x4 bw[KT][2];
    if constexpr (BIAS) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int g = 0; g < 2; ++g) bw[kt][g] = bw_ring[kt][g];
    }
    f32x16 s[KT], dp[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dp[kt][r] = dl;  // -D
        if constexpr (PRE) s[kt][r] = nl2;
      }
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4 ka = *(const u32x4*)(sK + kt * 32 * ROWB + to.rd(dc));
        const u32x4 va = *(const u32x4*)(sV + kt * 32 * ROWB + to.rd(dc));
        s[kt] = mfma32<BF16>(ka, qf[dc], s[kt]);
        pin_step<1, 1, FA_BWD_PIN_LA>(2 * (kt * DC + dc));
        dp[kt] = mfma32<BF16>(va, gf[dc], dp[kt]);
        pin_step<1, 1, FA_BWD_PIN_LA>(2 * (kt * DC + dc) + 1);
      }
    }
    pin_tail<1, FA_BWD_PIN_LA>();
    if constexpr (BIAS) {
      const float kb = PRE ? kLog2e : 1.0f / a.scale;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = bw[kt][g][e];
            s[kt][8 * g + 2 * e] = __builtin_fmaf(to_f32<BF16>((uint16_t)(w & 0xffffu)), kb, s[kt][8 * g + 2 * e]);
            s[kt][8 * g + 2 * e + 1] = __builtin_fmaf(to_f32<BF16>((uint16_t)(w >> 16)), kb, s[kt][8 * g + 2 * e + 1]);
          }
    }
    u32x4 ps[KC];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = PRE ? fast_exp2(s[kt][r]) : fast_exp2(__builtin_fmaf(s[kt][r], c, nl2));
        if constexpr (MASK) {
          // causal diagonal; with a bias also keys past N, whose bias entries
          // are read from the next row and must not reach dS
          const int keyi = k0 + kt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
          if ((CAUSAL && keyi > qrow) || (BIAS && keyi >= a.N)) p = 0.f;
        }
        dsv[r] = p * dp[kt][r];
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack2<BF16>(dsv[8 * g + 2 * e], dsv[8 * g + 2 * e + 1]);
        ps[2 * kt + g] = w;
      }
    }
    // dQ^T += K^T dS^T (rows: d with perm_o, cols: queries)
#pragma unroll
    for (int i = 0; i < DT * KC; ++i) {
      const int dt = FA_BWD_CHUNK_MAJOR ? i % DT : i / KC;
      const int kc = FA_BWD_CHUNK_MAJOR ? i / DT : i % KC;
      const u32x4 ka = tr_operand(sK, to.trl(dt), to.trh(dt), kc, ROWB);
      dqt[dt] = mfma32<BF16>(ka, ps[kc], dqt[dt]);
      pin_step<2, 2, FA_BWD_PIN_LA>(i);
    }
    pin_tail<2, FA_BWD_PIN_LA>();
  };

  // Bias ring load order: tile t's bias follows tile t - 1's K/V, so when
  // tile j's bias is read, the K/V of tiles j and j + 1 and tile j + 1's bias
  // are newer; at the end of iteration j only tile j + 2's bias is newer than
  // tile j + 1's K/V.
  constexpr int kTileLoads = 2 * LOADS;
  auto iteration = [&](int j, char* cur, char* nxt) {
    if constexpr (kBiasLds) {
      issue_tile(j + 1, nxt, j + 1 < n_kt);
      wait_vmem_keep<2 * kTileLoads + LB>();  // tile j's bias has landed
    } else {
      if (j + 1 < n_kt) issue_tile(j + 1, nxt);
    }
    const int k0 = j * BK;
    const bool active = !CAUSAL || (k0 <= qw0 + 31);
    u32x4 bw[KT][2];
    if constexpr (kBiasLds) {
      if (active) read_bias(j, bw);
      wait_lds();  // (the slot's reads have returned before it is refilled)
      issue_bias(j + 2, j + 2 < n_kt);
    }
    if (active) {
      if ((CAUSAL && k0 + BK - 1 > qw0) || (BIAS && k0 + BK > a.N)) {
        tile_body(std::true_type{}, cur, k0, bw);
      } else {
        tile_body(std::false_type{}, cur, k0, bw);
      }
    }
    if constexpr (kBiasLds) {
      wait_vmem_keep<LB>();
      barrier_no_fence();
    } else if constexpr (kCounted) {
      wait_vmem();
      barrier_no_fence();
    } else {
      wait_vmem();
      __syncthreads();
    }
  };

  char* st0 = smem;
  char* st1 = smem + STAGE;
  if constexpr (kBiasLds) {
    issue_bias(0, true);
    issue_tile(0, st0);
    issue_bias(1, 1 < n_kt);
    wait_vmem_keep<LB>();  // tile 0's K/V (and so tile 0's bias)
    barrier_no_fence();
  } else {
    issue_tile(0, st0);
    wait_vmem();
    if constexpr (kCounted) {
      barrier_no_fence();
    } else {
      __syncthreads();
    }
  }
  for (int j = 0; j < n_kt; j += 2) {
    iteration(j, st0, st1);
    if (j + 1 < n_kt) iteration(j + 1, st1, st0);
  }
  if constexpr (kBiasLds) wait_vmem();  // (the ring's loads past the end)

  const brsrc_t rdq = make_rsrc(a.dq + base, head_bytes);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const uint32_t off = ((uint32_t)qrow * D + dt * 32 + 16 * h) * 2u;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      u32x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        w[t] = pack2<BF16>(dqt[dt][8 * e + 2 * t] * a.scale, dqt[dt][8 * e + 2 * t + 1] * a.scale);
      bstore16(w, rdq, off + 16 * e, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename Kern>
hipError_t set_lds(Kern kern, int bytes) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

inline BwdArgs make_args(const BwdProblem& p) {
  BwdArgs a;
  a.bias = (const uint16_t*)p.bias;
  a.bias_sb = p.bias_sb;
  a.bias_sh = p.bias_sh;
  a.H = p.H;
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.dout = (const uint16_t*)p.dout;
  a.lse2 = p.lse2;
  a.delta = p.delta;
  a.dq = (uint16_t*)p.dq;
  a.dk = (uint16_t*)p.dk;
  a.dv = (uint16_t*)p.dv;
  a.N = p.N;
  a.BH = p.BH;
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  a.n_tiles = 0;
  return a;
}

template <int D, bool BF16, bool O_F32>
hipError_t launch_pre_t(const BwdProblem& p, hipStream_t stream) {
  const int rows = p.BH * p.N;
  constexpr int RPB = kBwdThreads / (D / 8);
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  hipLaunchKernelGGL((bwd_pre_kernel<D, BF16, O_F32>), grid, dim3(kBwdThreads), 0, stream, p.o,
                     (const uint16_t*)p.dout, p.lse, p.delta, p.lse2, rows);
  return hipGetLastError();
}

template <int D, bool BF16, bool CAUSAL, bool BIAS>
hipError_t launch_dkdv_t(const BwdProblem& p, hipStream_t stream) {
  BwdArgs a = make_args(p);
  a.n_tiles = (p.N + kDkvKeys - 1) / kDkvKeys;
  // two stages, then (bias) each wave's two-slot ring of BQ rows x 64 bytes
  constexpr int BQ = dkdv_bq<D, BF16, CAUSAL, BIAS>();
  const int lds = 2 * dkdv_stage_bytes<D, BQ>() + (BIAS ? (kBwdThreads / 64) * 2 * BQ * 64 : 0);
  auto kern = bwd_dkdv_kernel<D, BF16, CAUSAL, BIAS>;
  hipError_t e = set_lds(kern, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.BH * a.n_tiles)), dim3(kBwdThreads), lds, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16, bool CAUSAL, bool BIAS>
hipError_t launch_dq_t(const BwdProblem& p, hipStream_t stream) {
  BwdArgs a = make_args(p);
  a.n_tiles = (p.N + kDqRows - 1) / kDqRows;
  const int lds = 2 * dq_stage_bytes<D, BIAS>() + dq_ring_bytes<D, BIAS>();
  auto kern = bwd_dq_kernel<D, BF16, CAUSAL, BIAS>;
  hipError_t e = set_lds(kern, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.BH * a.n_tiles)), dim3(kBwdThreads), lds, stream, a);
  return hipGetLastError();
}

// Dispatch over the input type and either the O type (preprocess) or causal.
template <int D, template <int, bool, bool> class L>
hipError_t dispatch_d(const BwdProblem& p, hipStream_t s, bool third) {
  if (p.dtype < kF16 || p.dtype > kBF16OutF32) return hipErrorInvalidValue;
  const bool bf16 = p.dtype == kBF16 || p.dtype == kBF16OutF32;
  if (bf16) return third ? L<D, true, true>::run(p, s) : L<D, true, false>::run(p, s);
  return third ? L<D, false, true>::run(p, s) : L<D, false, false>::run(p, s);
}
template <int D, bool BF16, bool X>
struct PreL {
  static hipError_t run(const BwdProblem& p, hipStream_t s) { return launch_pre_t<D, BF16, X>(p, s); }
};
template <int D, bool BF16, bool X>
struct DkdvL {
  static hipError_t run(const BwdProblem& p, hipStream_t s) {
    return p.bias ? launch_dkdv_t<D, BF16, X, true>(p, s) : launch_dkdv_t<D, BF16, X, false>(p, s);
  }
};
template <int D, bool BF16, bool X>
struct DqL {
  static hipError_t run(const BwdProblem& p, hipStream_t s) {
    return p.bias ? launch_dq_t<D, BF16, X, true>(p, s) : launch_dq_t<D, BF16, X, false>(p, s);
  }
};

}  // namespace fa
