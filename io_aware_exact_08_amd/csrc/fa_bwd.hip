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
//  * bwd_pre   : D for every row (one pass over O and dO).
//  * bwd_dkdv  : a workgroup keeps 128 keys of K and V in registers (32 per
//                wave) and loops over 64-row query tiles streamed through LDS
//                (the loop order above); dK and dV accumulate in registers.
//  * bwd_dq    : a workgroup keeps 128 query rows of Q and dO in registers and
//                loops over 64-key K/V tiles streamed through LDS.
// All products use v_mfma_f32_32x32x16 with the same register-layout trick as
// the forward: the 32x32 accumulator of one product is, after rounding, the
// operand of the next, and tiles whose contraction runs over rows are stored
// transposed in LDS so each MFMA operand is one 16-byte read.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr int kBwdThreads = 256;

// ---------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool O_F32>
__global__ __launch_bounds__(kBwdThreads) void bwd_pre_kernel(const void* __restrict__ o,
                                                              const uint16_t* __restrict__ dout,
                                                              float* __restrict__ delta, int rows) {
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
  if (row < rows && c == 0) delta[row] = acc;
}

// LDS index helpers (16-bit element units).
template <int D>
__device__ __forceinline__ int rm_idx(int row, int chunk) {
  return row * D + ((chunk ^ swz_row(row)) * 8);
}
template <int BR>
__device__ __forceinline__ int tr_idx(int d, int col) {
  return d * BR + (((col >> 3) ^ swz_t(d)) * 8) + (col & 7);
}

// Write a row pair (rows 2kp, 2kp+1; 16-byte chunk c) row-major and, if
// requested, transposed into LDS tiles of BR rows.
template <int D, int BR, bool TRANSPOSED>
__device__ __forceinline__ void store_pair(uint16_t* rm, uint16_t* tr, int kp, int c, u32x4 r0, u32x4 r1) {
  const int kk = 2 * kp;
  *(u32x4*)(&rm[rm_idx<D>(kk, c)]) = r0;
  *(u32x4*)(&rm[rm_idx<D>(kk + 1, c)]) = r1;
  if constexpr (TRANSPOSED) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dd = c * 8 + e;
      const uint32_t w = (e & 1) ? hi_halves(r0[e >> 1], r1[e >> 1]) : lo_halves(r0[e >> 1], r1[e >> 1]);
      *(uint32_t*)(&tr[tr_idx<BR>(dd, kk)]) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup owns 128 keys (32 per wave); loop over 64-row query tiles.
// ---------------------------------------------------------------------------
constexpr int kDkvKeys = 128;  // keys per workgroup
constexpr int kDkvBQ = 64;     // query rows per streamed tile

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* delta;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int N;
  int BH;
  int n_tiles;  // workgroup tiles per head
  float c;      // scale * log2(e)
  float scale;
};

template <int D>
__host__ __device__ constexpr int dkdv_stage_elems() {
  // sQ, sQt, sdO, sdOt (16-bit) + LSE and D rows (float, 2 x 64 -> 256 halves)
  return 4 * kDkvBQ * D + 4 * kDkvBQ;
}

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BQ = kDkvBQ;
  constexpr int DC = D / 16;
  constexpr int DT = D / 32;
  constexpr int QT = BQ / 32;  // 32-row query tiles per streamed tile
  constexpr int QC = BQ / 16;  // 16-row query chunks (contraction of dK, dV)
  constexpr int CPR = D / 8;
  constexpr int PAIRS = (BQ / 2) * CPR / kBwdThreads;  // row pairs per thread per tensor
  static_assert(PAIRS * kBwdThreads == (BQ / 2) * CPR, "tile split");
  constexpr int STAGE = dkdv_stage_elems<D>();

  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

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
  const uint16_t* __restrict__ Qg = a.q + base;
  const uint16_t* __restrict__ dOg = a.dout + base;
  const float* __restrict__ Lg = a.lse + (size_t)bh * N;
  const float* __restrict__ Dg = a.delta + (size_t)bh * N;
  const int kw0 = kvt * kDkvKeys + wave * 32;  // first key of this wave
  const int key = kw0 + m;                     // this lane's key (column of S)

  // K and V fragments as B operands (lane: key m; slot i: d = 16dc + 8h + i).
  u32x4 kf[DC], vf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    if (key < N) {
      kf[dc] = *(const u32x4*)(a.k + base + (size_t)key * D + dc * 16 + 8 * h);
      vf[dc] = *(const u32x4*)(a.v + base + (size_t)key * D + dc * 16 + 8 * h);
    } else {
      kf[dc] = u32x4{0, 0, 0, 0};
      vf[dc] = u32x4{0, 0, 0, 0};
    }
  }

  f32x16 dkt[DT], dvt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dkt[dt] = f32x16{};
    dvt[dt] = f32x16{};
  }

  const int n_qt = (N + BQ - 1) / BQ;
  const int qt_begin = CAUSAL ? (kvt * kDkvKeys) / BQ : 0;

  u32x4 qreg[PAIRS][2], oreg[PAIRS][2];
  float lreg = 0.f;  // threads 0..63: LSE*log2e of one row; 64..127: D of one row

  auto load_tile = [&](int qt) {
    const int q0 = qt * BQ;
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
      const int p = tid + i * kBwdThreads;
      const int c = p % CPR, kp = p / CPR;
      const int r = q0 + 2 * kp;
      qreg[i][0] = r < N ? *(const u32x4*)(Qg + (size_t)r * D + c * 8) : u32x4{0, 0, 0, 0};
      qreg[i][1] = r + 1 < N ? *(const u32x4*)(Qg + (size_t)(r + 1) * D + c * 8) : u32x4{0, 0, 0, 0};
      oreg[i][0] = r < N ? *(const u32x4*)(dOg + (size_t)r * D + c * 8) : u32x4{0, 0, 0, 0};
      oreg[i][1] = r + 1 < N ? *(const u32x4*)(dOg + (size_t)(r + 1) * D + c * 8) : u32x4{0, 0, 0, 0};
    }
    if (tid < BQ) {
      const int r = q0 + tid;
      lreg = r < N ? Lg[r] * kLog2e : INFINITY;  // padded rows: P = exp2(-inf) = 0
    } else if (tid < 2 * BQ) {
      const int r = q0 + tid - BQ;
      lreg = r < N ? Dg[r] : 0.f;
    }
  };
  auto store_tile = [&](int st) {
    uint16_t* sQ = smem + st * STAGE;
    uint16_t* sQt = sQ + BQ * D;
    uint16_t* sdO = sQt + BQ * D;
    uint16_t* sdOt = sdO + BQ * D;
    float* sL = (float*)(sdOt + BQ * D);
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
      const int p = tid + i * kBwdThreads;
      const int c = p % CPR, kp = p / CPR;
      store_pair<D, BQ, true>(sQ, sQt, kp, c, qreg[i][0], qreg[i][1]);
      store_pair<D, BQ, true>(sdO, sdOt, kp, c, oreg[i][0], oreg[i][1]);
    }
    if (tid < 2 * BQ) sL[tid] = lreg;
  };

  if (qt_begin < n_qt) {
    load_tile(qt_begin);
    store_tile(0);
  }
  __syncthreads();

  const float c = a.c;
  for (int qt = qt_begin; qt < n_qt; ++qt) {
    const int st = (qt - qt_begin) & 1;
    if (qt + 1 < n_qt) load_tile(qt + 1);
    const int q0 = qt * BQ;
    const bool active = !CAUSAL || (q0 + BQ - 1 >= kw0);
    if (active) {
      const uint16_t* sQ = smem + st * STAGE;
      const uint16_t* sQt = sQ + BQ * D;
      const uint16_t* sdO = sQt + BQ * D;
      const uint16_t* sdOt = sdO + BQ * D;
      const float* sL = (const float*)(sdOt + BQ * D);
      const float* sD = sL + BQ;

      // S = Q K^T and dP = dO V^T (rows: queries with perm_k, cols: keys)
      f32x16 s[QT], dp[QT];
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        s[t] = f32x16{};
        dp[t] = f32x16{};
        const int row = t * 32 + perm_k(m);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const u32x4 qa = *(const u32x4*)(&sQ[rm_idx<D>(row, 2 * dc + h)]);
          const u32x4 ga = *(const u32x4*)(&sdO[rm_idx<D>(row, 2 * dc + h)]);
          s[t] = mfma32<BF16>(qa, kf[dc], s[t]);
          dp[t] = mfma32<BF16>(ga, vf[dc], dp[t]);
        }
      }
      const bool need_mask = (kw0 + 32 > N) || (CAUSAL && q0 < kw0 + 31);
      u32x4 pp[QC], ps[QC];
#pragma unroll
      for (int t = 0; t < QT; ++t) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          // register r = 8g + e  <->  query row t*32 + 16g + 8h + e of the tile
          const int qb = t * 32 + 16 * g + 8 * h;
          const f32x4 l0 = *(const f32x4*)(&sL[qb]);
          const f32x4 l1 = *(const f32x4*)(&sL[qb + 4]);
          const f32x4 d0 = *(const f32x4*)(&sD[qb]);
          const f32x4 d1 = *(const f32x4*)(&sD[qb + 4]);
          float pv[8], dsv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float lse2 = e < 4 ? l0[e] : l1[e - 4];
            const float dd = e < 4 ? d0[e] : d1[e - 4];
            float p = fast_exp2(__builtin_fmaf(s[t][8 * g + e], c, -lse2));
            if (need_mask) {
              const int qrow = q0 + qb + e;
              if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
            }
            pv[e] = p;
            dsv[e] = p * (dp[t][8 * g + e] - dd);
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
      }
      // dV^T += dO^T P ; dK^T += Q^T dS   (rows: d with perm_o, cols: keys)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int drow = dt * 32 + perm_o(m);
#pragma unroll
        for (int qc = 0; qc < QC; ++qc) {
          const int col = 16 * qc + 8 * h;
          const u32x4 ga = *(const u32x4*)(&sdOt[tr_idx<BQ>(drow, col)]);
          const u32x4 qa = *(const u32x4*)(&sQt[tr_idx<BQ>(drow, col)]);
          dvt[dt] = mfma32<BF16>(ga, pp[qc], dvt[dt]);
          dkt[dt] = mfma32<BF16>(qa, ps[qc], dkt[dt]);
        }
      }
    }
    if (qt + 1 < n_qt) store_tile(st ^ 1);
    __syncthreads();
  }

  if (key < N) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const size_t off = base + (size_t)key * D + dt * 32 + 16 * h;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        u32x4 wk, wv;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          wk[t] = pack2<BF16>(dkt[dt][8 * e + 2 * t] * a.scale, dkt[dt][8 * e + 2 * t + 1] * a.scale);
          wv[t] = pack2<BF16>(dvt[dt][8 * e + 2 * t], dvt[dt][8 * e + 2 * t + 1]);
        }
        *(u32x4*)(a.dk + off + 8 * e) = wk;
        *(u32x4*)(a.dv + off + 8 * e) = wv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup owns 128 query rows (32 per wave); loop over 64-key tiles.
// ---------------------------------------------------------------------------
constexpr int kDqRows = 128;
constexpr int kDqBK = 64;

template <int D>
__host__ __device__ constexpr int dq_stage_elems() {
  return 3 * kDqBK * D;  // sK, sKt, sV
}

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BK = kDqBK;
  constexpr int DC = D / 16;
  constexpr int DT = D / 32;
  constexpr int KT = BK / 32;
  constexpr int KC = BK / 16;
  constexpr int CPR = D / 8;
  constexpr int PAIRS = (BK / 2) * CPR / kBwdThreads;
  static_assert(PAIRS * kBwdThreads == (BK / 2) * CPR, "tile split");
  constexpr int STAGE = dq_stage_elems<D>();

  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

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
  const uint16_t* __restrict__ Kg = a.k + base;
  const uint16_t* __restrict__ Vg = a.v + base;
  const int qw0 = qt * kDqRows + wave * 32;
  const int qrow = qw0 + m;

  u32x4 qf[DC], gf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    if (qrow < N) {
      qf[dc] = *(const u32x4*)(a.q + base + (size_t)qrow * D + dc * 16 + 8 * h);
      gf[dc] = *(const u32x4*)(a.dout + base + (size_t)qrow * D + dc * 16 + 8 * h);
    } else {
      qf[dc] = u32x4{0, 0, 0, 0};
      gf[dc] = u32x4{0, 0, 0, 0};
    }
  }
  const float lse2 = qrow < N ? a.lse[(size_t)bh * N + qrow] * kLog2e : INFINITY;
  const float dl = qrow < N ? a.delta[(size_t)bh * N + qrow] : 0.f;

  f32x16 dqt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqt[dt] = f32x16{};

  const int kend = CAUSAL ? min(N, qt * kDqRows + kDqRows) : N;
  const int n_kt = (kend + BK - 1) / BK;

  u32x4 kreg[PAIRS][2], vreg[PAIRS][2];
  auto load_tile = [&](int j) {
    const int k0 = j * BK;
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
      const int p = tid + i * kBwdThreads;
      const int c = p % CPR, kp = p / CPR;
      const int r = k0 + 2 * kp;
      kreg[i][0] = r < N ? *(const u32x4*)(Kg + (size_t)r * D + c * 8) : u32x4{0, 0, 0, 0};
      kreg[i][1] = r + 1 < N ? *(const u32x4*)(Kg + (size_t)(r + 1) * D + c * 8) : u32x4{0, 0, 0, 0};
      vreg[i][0] = r < N ? *(const u32x4*)(Vg + (size_t)r * D + c * 8) : u32x4{0, 0, 0, 0};
      vreg[i][1] = r + 1 < N ? *(const u32x4*)(Vg + (size_t)(r + 1) * D + c * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int st) {
    uint16_t* sK = smem + st * STAGE;
    uint16_t* sKt = sK + BK * D;
    uint16_t* sV = sKt + BK * D;
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
      const int p = tid + i * kBwdThreads;
      const int c = p % CPR, kp = p / CPR;
      store_pair<D, BK, true>(sK, sKt, kp, c, kreg[i][0], kreg[i][1]);
      store_pair<D, BK, false>(sV, nullptr, kp, c, vreg[i][0], vreg[i][1]);
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const float c = a.c;
  for (int j = 0; j < n_kt; ++j) {
    const int st = j & 1;
    if (j + 1 < n_kt) load_tile(j + 1);
    const int k0 = j * BK;
    const bool active = !CAUSAL || (k0 <= qw0 + 31);
    if (active) {
      const uint16_t* sK = smem + st * STAGE;
      const uint16_t* sKt = sK + BK * D;
      const uint16_t* sV = sKt + BK * D;
      // S^T = K Q^T, dP^T = V dO^T (rows: keys with perm_k, cols: queries)
      f32x16 s[KT], dp[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = f32x16{};
        dp[kt] = f32x16{};
        const int row = kt * 32 + perm_k(m);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const u32x4 ka = *(const u32x4*)(&sK[rm_idx<D>(row, 2 * dc + h)]);
          const u32x4 va = *(const u32x4*)(&sV[rm_idx<D>(row, 2 * dc + h)]);
          s[kt] = mfma32<BF16>(ka, qf[dc], s[kt]);
          dp[kt] = mfma32<BF16>(va, gf[dc], dp[kt]);
        }
      }
      const bool need_mask = (k0 + BK > N) || (CAUSAL && k0 + BK - 1 > qw0);
      u32x4 ps[KC];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        float dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[kt][r], c, -lse2));
          if (need_mask) {
            const int key = k0 + kt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
            if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
          }
          dsv[r] = p * (dp[kt][r] - dl);
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
      for (int dt = 0; dt < DT; ++dt) {
        const int drow = dt * 32 + perm_o(m);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const u32x4 ka = *(const u32x4*)(&sKt[tr_idx<BK>(drow, 16 * kc + 8 * h)]);
          dqt[dt] = mfma32<BF16>(ka, ps[kc], dqt[dt]);
        }
      }
    }
    if (j + 1 < n_kt) store_tile(st ^ 1);
    __syncthreads();
  }

  if (qrow < N) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const size_t off = base + (size_t)qrow * D + dt * 32 + 16 * h;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w[t] = pack2<BF16>(dqt[dt][8 * e + 2 * t] * a.scale, dqt[dt][8 * e + 2 * t + 1] * a.scale);
        *(u32x4*)(a.dq + off + 8 * e) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename Kern>
static hipError_t set_lds(Kern kern, int bytes) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int D, bool BF16, bool O_F32, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdProblem& p, hipStream_t stream) {
  const int rows = p.BH * p.N;
  {
    constexpr int RPB = kBwdThreads / (D / 8);
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    hipLaunchKernelGGL((bwd_pre_kernel<D, BF16, O_F32>), grid, dim3(kBwdThreads), 0, stream, p.o,
                       (const uint16_t*)p.dout, p.delta, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs a;
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.dout = (const uint16_t*)p.dout;
  a.lse = p.lse;
  a.delta = p.delta;
  a.dq = (uint16_t*)p.dq;
  a.dk = (uint16_t*)p.dk;
  a.dv = (uint16_t*)p.dv;
  a.N = p.N;
  a.BH = p.BH;
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  {
    a.n_tiles = (p.N + kDkvKeys - 1) / kDkvKeys;
    const int lds = 2 * dkdv_stage_elems<D>() * 2;
    auto kern = bwd_dkdv_kernel<D, BF16, CAUSAL>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.BH * a.n_tiles)), dim3(kBwdThreads), lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    a.n_tiles = (p.N + kDqRows - 1) / kDqRows;
    const int lds = 2 * dq_stage_elems<D>() * 2;
    auto kern = bwd_dq_kernel<D, BF16, CAUSAL>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.BH * a.n_tiles)), dim3(kBwdThreads), lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D, bool BF16, bool O_F32>
static hipError_t launch_bwd_c(const BwdProblem& p, hipStream_t s) {
  return p.causal ? launch_bwd_t<D, BF16, O_F32, true>(p, s) : launch_bwd_t<D, BF16, O_F32, false>(p, s);
}

template <int D>
static hipError_t launch_bwd_d(const BwdProblem& p, hipStream_t s) {
  switch (p.dtype) {
    case kF16: return launch_bwd_c<D, false, false>(p, s);
    case kBF16: return launch_bwd_c<D, true, false>(p, s);
    case kF16OutF32: return launch_bwd_c<D, false, true>(p, s);
    case kBF16OutF32: return launch_bwd_c<D, true, true>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdProblem& p, hipStream_t s) {
  if (p.d == 64) return launch_bwd_d<64>(p, s);
  if (p.d == 128) return launch_bwd_d<128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
