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
//  * K tiles sit row-major in LDS; V tiles are transposed to [d][key] while
//    being written to LDS so the V^T operand is one 16-byte read per lane.
//    Both are double-buffered: tile j+1 is fetched from HBM into registers
//    while tile j is multiplied, then written to the other LDS buffer.
//  * fp16 rescaling is lazy: the running max used in the exponent is only
//    raised when a row's new max exceeds it by more than 8 (log2 units).  Any
//    common reference value gives the same O = acc / l and LSE = m + log2 l
//    exactly; the bound keeps every probability below 2^8 so nothing
//    overflows.  bf16 rescales whenever the max grows (see threshold below).
//  * O is normalised by the sum of the probabilities as rounded for the P V
//    product (one v_dot2 per pair), so numerator and denominator carry the
//    same rounding and a dominant key's rounding error cancels.  The fp16
//    path also takes its LSE from that sum (rounding moves it by at most
//    2^-11 relative, i.e. < 5e-4 in LSE); the bf16 path keeps a second,
//    fp32 sum of the unrounded probabilities for the LSE, where a bf16 sum
//    could be off by 2^-9.
//  * Non-causal launches remap workgroup ids so that all query tiles of a head
//    run on one XCD (consecutive ids are dealt round-robin over the 8 XCDs),
//    keeping that head's K/V in one L2.  Causal launches issue the heaviest
//    (last) query tiles first.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct FwdCfg;
template <>
struct FwdCfg<64> {
  static constexpr int QB = 2;   // 32-row query blocks per wave
  static constexpr int BK = 64;  // keys per tile
};
template <>
struct FwdCfg<128> {
  static constexpr int QB = 1;
  static constexpr int BK = 64;
};

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// Lazy-rescale threshold (log2 units).  bf16 keeps the exact running max
// (threshold 0): the dominant probability is then exactly 1 and is not
// rounded, which matters with 8-bit mantissas when one key dominates a row.
template <bool BF16>
constexpr float rescale_threshold() { return BF16 ? 0.0f : 8.0f; }

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
};

template <int D, bool BF16, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a) {
  constexpr int QB = FwdCfg<D>::QB;
  constexpr int BK = FwdCfg<D>::BK;
  constexpr int BQ = kWaves * QB * 32;
  constexpr int DC = D / 16;  // 16-wide d chunks (contraction of S^T)
  constexpr int DT = D / 32;  // 32-row d tiles of O^T
  constexpr int KT = BK / 32; // 32-row key tiles of S^T
  constexpr int KC = BK / 16; // 16-key chunks (contraction of O^T)
  constexpr int CPR = D / 8;  // 16-byte chunks per K row
  constexpr int K_LOADS = BK * CPR / kThreads;        // 16B K chunks per thread
  constexpr int V_LOADS = (BK / 2) * CPR / kThreads;  // row pairs per thread
  static_assert(K_LOADS * kThreads == BK * CPR, "K tile split");
  static_assert(V_LOADS * kThreads == (BK / 2) * CPR, "V tile split");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BK * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * BK];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 31;
  const int h = lane >> 5;

  int bh, qt;
  {
    const int bid = blockIdx.x;
    if (CAUSAL) {
      qt = a.n_qtiles - 1 - bid / a.BH;
      bh = bid % a.BH;
    } else {
      const int G = gridDim.x;
      const int lin = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
      bh = lin / a.n_qtiles;
      qt = lin % a.n_qtiles;
    }
  }
  const int N = a.N;
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qg = a.q + base;
  const uint16_t* __restrict__ Kg = a.k + base;
  const uint16_t* __restrict__ Vg = a.v + base;
  const int qw0 = qt * BQ + wave * (QB * 32);  // first query row of this wave

  // Q^T fragments (B operand of S^T = K Q^T): lane (query m, half h), slot i
  // holds d = 16*dc + 8*h + i.
  u32x4 qf[QB][DC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + m;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (row < N) {
        qf[qb][dc] = *(const u32x4*)(Qg + (size_t)row * D + dc * 16 + 8 * h);
      } else {
        qf[qb][dc] = u32x4{0, 0, 0, 0};
      }
    }
  }

  const int kend = CAUSAL ? min(N, qt * BQ + BQ) : N;
  const int n_kt = (kend + BK - 1) / BK;

  u32x4 kreg[K_LOADS];
  u32x4 vreg[V_LOADS][2];

  auto load_tile = [&](int j) {
    const int k0 = j * BK;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int g = tid + i * kThreads;
      const int row = g / CPR, c = g % CPR;
      const int key = k0 + row;
      kreg[i] = key < N ? *(const u32x4*)(Kg + (size_t)key * D + c * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int p = tid + i * kThreads;
      const int c = p % CPR, kp = p / CPR;
      const int key = k0 + 2 * kp;
      vreg[i][0] = key < N ? *(const u32x4*)(Vg + (size_t)key * D + c * 8) : u32x4{0, 0, 0, 0};
      vreg[i][1] = key + 1 < N ? *(const u32x4*)(Vg + (size_t)(key + 1) * D + c * 8)
                               : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int g = tid + i * kThreads;
      const int row = g / CPR, c = g % CPR;
      *(u32x4*)(&sK[st][row * D + ((c ^ swz_row(row)) * 8)]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int p = tid + i * kThreads;
      const int c = p % CPR, kp = p / CPR;
      const int kk = 2 * kp;  // key offset inside the tile (even)
      const u32x4 r0 = vreg[i][0], r1 = vreg[i][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = c * 8 + e;
        const uint32_t w = (e & 1) ? hi_halves(r0[e >> 1], r1[e >> 1])
                                   : lo_halves(r0[e >> 1], r1[e >> 1]);
        *(uint32_t*)(&sV[st][dd * BK + (((kk >> 3) ^ swz_t(dd)) * 8) + (kk & 7)]) = w;
      }
    }
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

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const float c = a.c;
  for (int j = 0; j < n_kt; ++j) {
    const int st = j & 1;
    if (j + 1 < n_kt) load_tile(j + 1);
    const int k0 = j * BK;
    const bool active = !CAUSAL || (k0 <= qw0 + QB * 32 - 1);
    if (active) {
      // ---- S^T = K Q^T -------------------------------------------------
      f32x16 s[QB][KT];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) s[qb][kt] = f32x16{};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int row = kt * 32 + perm_k(m);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const u32x4 af = *(const u32x4*)(&sK[st][row * D + (((2 * dc + h) ^ swz_row(row)) * 8)]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kt] = mfma32<BF16>(af, qf[qb][dc], s[qb][kt]);
        }
      }
      // ---- masks (tail keys; causal diagonal) ---------------------------
      const bool need_mask = (k0 + BK > N) || (CAUSAL && k0 + BK - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qrow = qw0 + qb * 32 + m;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
              if (key >= N || (CAUSAL && key > qrow)) s[qb][kt][r] = -INFINITY;
            }
        }
      }
      // ---- online softmax ------------------------------------------------
      u32x4 pf[QB][KC];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kt][r]);
        mx = max_halves(mx);
        const float mnew = mx * c;
        const bool grow = mnew > m_run[qb] + rescale_threshold<BF16>();
        if (__ballot(grow) != 0ull) {
          // Only rows that grew move their reference (the others get alpha = 1
          // exactly), so every row's result depends on that row's data alone.
          const float mn = grow ? mnew : m_run[qb];
          const float alpha = (m_run[qb] == -INFINITY) ? 0.f : fast_exp2(m_run[qb] - mn);
          m_run[qb] = mn;
          l_run[qb] *= alpha;
          if constexpr (BF16) l32_run[qb] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[qb][dt] *= alpha;
        }
        const float neg_m = -m_run[qb];
        float lsum = 0.f, lsum32 = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = fast_exp2(__builtin_fmaf(s[qb][kt][r], c, neg_m));
            if constexpr (BF16) lsum32 += p[r];
          }
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] = pack2<BF16>(p[8 * half + 2 * e], p[8 * half + 2 * e + 1]);
              lsum = sum2<BF16>(w[e], lsum);
            }
            pf[qb][2 * kt + half] = w;
          }
        }
        l_run[qb] += lsum;
        if constexpr (BF16) l32_run[qb] += lsum32;
      }
      // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int drow = dt * 32 + perm_o(m);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const u32x4 vf = *(const u32x4*)(&sV[st][drow * BK + (((2 * kc + h) ^ swz_t(drow)) * 8)]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][dt] = mfma32<BF16>(vf, pf[qb][kc], oacc[qb][dt]);
        }
      }
    }
    if (j + 1 < n_kt) store_tile(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + m;
    // cross-half sums outside any divergent branch (all 64 lanes take part)
    const float lt = sum_halves(l_run[qb]);
    const float ll = BF16 ? sum_halves(l32_run[qb]) : lt;
    if (row < N) {
      const float inv = 1.0f / lt;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const size_t off = base + (size_t)row * D + dt * 32 + 16 * h;
        if constexpr (OUT_F32) {
          float* op = (float*)a.o + off;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f32x4 w;
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] = oacc[qb][dt][4 * e + t] * inv;
            *(f32x4*)(op + 4 * e) = w;
          }
        } else {
          uint16_t* op = (uint16_t*)a.o + off;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            u32x4 w;
#pragma unroll
            for (int t = 0; t < 4; ++t)
              w[t] = pack2<BF16>(oacc[qb][dt][8 * e + 2 * t] * inv, oacc[qb][dt][8 * e + 2 * t + 1] * inv);
            *(u32x4*)(op + 8 * e) = w;
          }
        }
      }
      if (h == 0) {
        a.lse[(size_t)bh * N + row] = (m_run[qb] + fast_log2(ll)) * kLn2;
      }
    }
  }
}

template <int D, bool BF16, bool CAUSAL, bool OUT_F32>
static hipError_t launch_fwd_t(const FwdProblem& p, hipStream_t stream) {
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
  const dim3 grid((unsigned)(a.BH * a.n_qtiles));
  hipLaunchKernelGGL((fwd_kernel<D, BF16, CAUSAL, OUT_F32>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16, bool OUT_F32>
static hipError_t launch_fwd_c(const FwdProblem& p, hipStream_t s) {
  return p.causal ? launch_fwd_t<D, BF16, true, OUT_F32>(p, s) : launch_fwd_t<D, BF16, false, OUT_F32>(p, s);
}

template <int D>
static hipError_t launch_fwd_d(const FwdProblem& p, hipStream_t s) {
  switch (p.dtype) {
    case kF16: return launch_fwd_c<D, false, false>(p, s);
    case kBF16: return launch_fwd_c<D, true, false>(p, s);
    case kF16OutF32: return launch_fwd_c<D, false, true>(p, s);
    case kBF16OutF32: return launch_fwd_c<D, true, true>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd(const FwdProblem& p, hipStream_t s) {
  if (p.d == 64) return launch_fwd_d<64>(p, s);
  if (p.d == 128) return launch_fwd_d<128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
