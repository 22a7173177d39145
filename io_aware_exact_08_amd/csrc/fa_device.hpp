// Device-side building blocks for the gfx950 attention kernels: operand
// vector types, the 32x32x16 MFMA, RNE pair conversion, LDS swizzles and the
// register-layout permutations that let the score accumulator feed the P.V
// product without an LDS round trip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// C[32x32] += A[32x16] * B[16x32], fp32 accumulate.  Lane l supplies row (l%32)
// of A and column (l%32) of B, eight k-values each; lanes l and l+32 supply
// complementary k-halves.  A k-slot of A pairs with the same k-slot of B, so
// any consistent assignment of physical indices to slots gives the same sum.
// Output: lane l holds column l%32, register r holds row 8*(r/4)+4*(l/32)+r%4.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// C[16x16] += A[16x32] * B[32x16], fp32 accumulate.  Lane l supplies row
// (l%16) of A and column (l%16) of B, eight k-values each (k = 8(l/16) + i);
// lane l receives column l%16, rows 4(l/16) .. 4(l/16)+3.
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Raw buffer access.  A resource covers [base, base + bytes); loads outside it
// return 0 and stores outside it are dropped by the hardware, which handles
// ragged tails without branches.
typedef __amdgpu_buffer_rsrc_t brsrc_t;
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit data format

__device__ __forceinline__ brsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ u32x4 bload16(brsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void bstore16(u32x4 v, brsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v),
                                         r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void bstore8(u32x2 v, brsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void bstore4(float v, brsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
}

// Direct buffer -> LDS load of 16 bytes per lane: lane l of the wave writes
// lds_base + 16*l (lds_base must be wave-uniform); out-of-range reads land as
// zeros.  Completion is tracked by vmcnt, see wait_vmem().
__device__ __forceinline__ void bload16_lds(brsrc_t r, void* lds_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           (int)voff, (int)soff, 0, 0);
}
// The same direct load written as inline assembly, for pipelines that count
// every wait themselves.  The compiler does not see it, so it neither holds
// later LDS reads behind it (it cannot tell which LDS stage a read touches,
// and would wait for every direct load in flight) nor counts it in its own
// vmcnt waits: a kernel that uses it must issue no other vector-memory load
// whose result the compiler waits for while these are in flight.  `rs` is the
// four-word resource (wave-uniform), `lds` the wave's LDS byte address (form
// it as an integer from the __shared__ array, not from a generic pointer,
// which the compiler would keep in a register pair).
// Nothing is written to registers, so nothing in flight can be overwritten.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), (uint32_t)kBufferFlags};
}
// (m0, which the instruction takes its LDS address from, is restored: the
// compiler may keep a value of its own there)
__device__ __forceinline__ void bload16_lds_asm(const u32x4& rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
      : "memory");
}
// Workgroup barrier for pipelines whose direct loads are counted by hand:
// this wave's LDS reads have returned (so no stage it read can be refilled
// under them) and the compiler keeps LDS accesses on their side of it; the
// caller has already waited (vmcnt) for the loads the other waves will read.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Make the compiler wait here for a value it loaded (an empty asm that reads
// it).  Kernels with hand-counted loads call it on their compiler-visible
// loads before the loop: left to the first use inside the loop, the
// compiler's wait would count none of the hand-counted loads and drain them.
template <typename T>
__device__ __forceinline__ void settle(const T& v) { asm volatile("" ::"v"(v)); }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most K vector-memory operations of this wave are outstanding.
template <int K>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(K >= 0 && K < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte rows loaded by lanes
// 4*j + i/4, j = 0..3 (element j of the result).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_byte_addr) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)lds_byte_addr));
  return __builtin_bit_cast(u32x2, v);
}

// The same read at a 32-bit LDS byte address.  A caller that keeps a
// per-lane base in a register and adds a constant below 2^16 gets the
// constant folded into the instruction's offset field.
__device__ __forceinline__ u32x2 lds_read_tr16_at(uint32_t lds_byte_addr) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)lds_byte_addr);
  return __builtin_bit_cast(u32x2, v);
}

// Two floats -> two 16-bit values in one dword, round-to-nearest-even.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (BF16) {
    bf16x2 v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v;
    v.x = (_Float16)lo;
    v.y = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t bits) {
  if constexpr (BF16) {
    return __uint_as_float(((uint32_t)bits) << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
}

// acc + lo + hi of a packed pair of 16-bit values (v_dot2c_f32_{f16,bf16}
// against (1, 1)): the products are exact, the sum is in fp32.
template <bool BF16>
__device__ __forceinline__ float sum2(uint32_t w, float acc) {
  if constexpr (BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3C003C00u),
                                  acc, false);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine a value with the one held by lane l^32 (the other half of the
// wave) using v_permlane32_swap: with both operands x, lane l < 32 receives
// (x_l, x_{l+32}) and lane l >= 32 receives (x_{l-32}, x_l).  The max and the
// (commutative) sum are then identical in both halves.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The value of lane l ^ 16 (ds_swizzle in bit mode: and 0x1f, or 0, xor 0x10,
// within each 32-lane half).
__device__ __forceinline__ float swap16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401f));
}
// Max and sum over lanes l, l^16, l^32, l^48 (identical in all four).
__device__ __forceinline__ float max4(float x) { return max_halves(fmaxf(x, swap16(x))); }
__device__ __forceinline__ float sum4(float x) { return sum_halves(x + swap16(x)); }

// Row permutation applied when loading the A operand of a 32x32 MFMA so that
// the output's register r of lane half h maps to row 16*(r/8) + 8*h + r%8:
// each lane then holds, per 16-row chunk, eight consecutive rows - exactly the
// k-slots of the next MFMA's operand.  (Swaps bits 2 and 3 of the row.)
__device__ __forceinline__ int perm_k(int m) {
  return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// Row permutation so that output register r of lane half h maps to row
// 16*h + r: each lane holds sixteen consecutive rows (contiguous stores).
__device__ __forceinline__ int perm_o(int m) {
  return (((m >> 2) & 1) << 4) | ((m >> 3) << 2) | (m & 3);
}

// 16-byte-chunk XOR swizzles for row-major LDS tiles of D 16-bit columns
// (chunk c of tile row r is stored at chunk position c ^ swz(r)).
//
// gfx950 LDS has 64 banks of 4 bytes, i.e. a 256-byte bank window: a d=64 row
// (128 B) shares its window with its neighbour of opposite parity, a d=128 row
// fills one window.  ds_read_b128 serves 16 consecutive lanes per cycle and
// ds_read_b64 (also the transposing form) 32, so a read is conflict-free when
// those lanes land on distinct 16-byte slots of the window.
//  - Row operand (rows perm_k(m), one chunk per instruction): the 16 lanes of
//    a cycle cover all row residues mod 16, so the XOR must be a bijection of
//    row bits 1..3 (d=64: bit 0 picks the window half) or of bits 0..3 (d=128).
//  - Transposing read (lanes on rows 8h + j, j < 4, four chunks 4t..4t+3):
//    the 32 lanes of a cycle cover row bits 0 and 1, so the XOR must move the
//    four-chunk block by row bit 1 (d=64) or by row bits 0 and 1 (d=128).

// Tiles read only as a row operand, or both ways.  The XOR depends on row bit 2,
// so a transposing read of rows r + 4 needs its own per-lane offset.
template <int D>
__device__ __forceinline__ int swz_dual(int r) {
  if constexpr (D == 64)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 1) | (((r >> 3) & 1) << 1);
  else
    return ((r & 1) << 2) | (((r >> 1) & 1) << 3) | ((r >> 2) & 1) | (((r >> 3) & 1) << 1);
}
// Tiles read only through the transposing read: the XOR depends on row bits 0
// and 1 alone, so rows r and r + 4 share one per-lane offset.
template <int D>
__device__ __forceinline__ int swz_tr(int r) {
  if constexpr (D == 64)
    return (r & 1) | (((r >> 1) & 1) << 2);
  else
    return ((r & 1) << 2) | (((r >> 1) & 1) << 3);
}

// Operand-read placement for a chain of MFMAs that each take R LDS reads:
// the reads of the first LA MFMAs go first, then each MFMA is followed by the
// reads of the one LA places later.  Left free, the scheduler can hoist every
// read of a chain ahead of it (for the d=256 forward with one wave per SIMD,
// 128 registers, since it counts the accumulation registers as headroom).
// A scheduling group fills from the instructions before its barrier, so
// pin_step(i) follows the code of MFMA i (i counted from 0 along the chain)
// and pin_tail the chain; `sync` separates chains in one scheduling region.
template <int sync, int R, int LA>
__device__ __forceinline__ void pin_step(int i) {
  if (i == LA - 1) {
    __builtin_amdgcn_sched_group_barrier(0x100, R * LA, sync);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, sync);
  } else if (i >= LA) {
    __builtin_amdgcn_sched_group_barrier(0x100, R, sync);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, sync);
  }
}
template <int sync, int LA>
__device__ __forceinline__ void pin_tail() {
#pragma unroll
  for (int i = 1; i < LA; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, sync);
}

}  // namespace fa
