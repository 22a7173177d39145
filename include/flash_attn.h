/*
 * flash_attn.h - C ABI of the MI355X (gfx950) exact-attention library.
 *
 * Operation (page 1, examples 1-3; page 2, "Kernel Fusion" and "Tiling"):
 *     O = softmax(scale * Q K^T) V          softmax over the key axis
 * computed exactly (not approximated) by one fused kernel that streams K/V
 * tiles through on-chip memory under an online softmax, and the backward of
 * page 2, "Re-computation", which rebuilds the probabilities blockwise from the
 * saved row log-sum-exp instead of storing the N x N matrix.
 *
 * Conventions shared by every entry point
 *  - Layout: Q, K, V, O, dO, dQ, dK, dV are dense row-major [B, H, N, d] with d
 *    innermost (element (b,h,i,c) at ((b*H + h)*N + i)*d + c), the layout of
 *    page 1, example 2.  LSE is [B, H, N] float32.
 *  - Pointers are DEVICE pointers (HIP global memory) of the calling process's
 *    current device.  Every tensor pointer must be 16-byte aligned.
 *  - Ownership: the caller allocates and frees every buffer.  The library never
 *    allocates device memory.  Its only global state belongs to
 *    flash_attn_bwd_noalloc: a static device array and the per-device address
 *    of it, set once under a lock.  Calls are thread-safe (apart from that
 *    entry point's shared array, see there).  Inputs are read-only; outputs
 *    are fully overwritten.
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and the call returns before it runs.  Faults inside the kernels
 *    surface at the caller's next synchronisation.
 *  - Errors: the return value is a fa_status.  Arguments are validated before
 *    anything is enqueued; on a non-zero status nothing was launched.
 *  - Sizes: B, H, N >= 1, any N (tail tiles are masked); head dimension d in
 *    {64, 128, 256} (page 2, "工程落地的关键考量", hardware requirements,
 *    names 64, 128 and 256 as the preferred head sizes); B*H*N*d < 2^31
 *    elements per tensor, and
 *    (N + 256) * d * s < 2^32 bytes for every per-head output with elements
 *    of s bytes (s = 4 for a float32 O and for the split-KV partials, 2 for
 *    16-bit O, dQ, dK, dV): the kernels address a head through a 32-bit byte
 *    range, including the dropped stores of a ragged last tile.  Shapes
 *    beyond either limit return FA_ERR_SHAPE before anything is launched.
 *  - Causal: key j is visible to query i iff j <= i (queries and keys share the
 *    same length N).
 *  - Arithmetic: fp16 or bf16 operands, float32 accumulation and softmax state,
 *    probabilities rounded to the operand type (round-to-nearest-even) before
 *    the P V product.
 */
#ifndef FLASH_ATTN_H_
#define FLASH_ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL                       */
  FA_ERR_SHAPE = 2,     /* B, H or N < 1, a tensor of 2^31 elements or more,
                           a per-head output range of 2^32 bytes or more, or
                           causal not 0/1                                     */
  FA_ERR_HEADDIM = 3,   /* d not in {64,128,256}                            */
  FA_ERR_DTYPE = 4,     /* unknown fa_dtype                                 */
  FA_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned                 */
  FA_ERR_LAUNCH = 6,    /* the HIP runtime rejected a kernel launch         */
  FA_ERR_WORKSPACE = 7, /* workspace missing or too small                   */
  FA_ERR_SCALE = 8,     /* scale is not a finite positive number            */
  FA_ERR_SPLITS = 9,    /* num_splits outside [0, 64]                       */
  FA_ERR_SCRATCH = 10   /* flash_attn_bwd_noalloc: the problem's workspace
                           exceeds FA_NOALLOC_SCRATCH_BYTES                  */
} fa_status;

/* Element types: Q/K/V (and dQ/dK/dV) type x O (and dO) type. */
typedef enum {
  FA_F16 = 0,          /* fp16 in, fp16 O                                   */
  FA_BF16 = 1,         /* bf16 in, bf16 O                                   */
  FA_F16_OUT_F32 = 2,  /* fp16 in, float32 O                                */
  FA_BF16_OUT_F32 = 3  /* bf16 in, float32 O                                */
} fa_dtype;

/*
 * Forward.  Page 2, "Kernel Fusion" (one kernel; only the output reaches
 * global memory) and "Tiling" (B_q x B_k tiles, online softmax: per-tile max
 * and exp-sum, running max update with rescaled normaliser, one final
 * normalisation).
 *
 *   q, k, v : [B,H,N,d] of the input type (read)
 *   o       : [B,H,N,d] of the output type (written)
 *   lse     : [B,H,N] float32 (written), LSE_i = ln sum_{j visible}
 *             exp(scale * q_i . k_j), natural log with the scale included; the
 *             backward rebuilds P_ij = exp(scale * q_i . k_j - LSE_i) from it.
 *   scale   : finite, > 0 (usually 1/sqrt(d))
 *   causal  : 0 or 1
 *   dtype   : fa_dtype
 *   stream  : hipStream_t
 */
int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   void* stream);

/*
 * Backward.  Page 2, "Re-computation": scores are not cached; P is recomputed
 * per tile from Q, K and the forward's LSE.  Gradients of L = <dO, O>:
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
 *   dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * Three kernels on `stream`: -D and -LSE*log2(e) (one pass over O, dO and LSE),
 * dK/dV (each workgroup keeps a K/V tile and loops over query tiles, the loop
 * order of that section), dQ (each workgroup keeps a query tile and loops
 * over K/V tiles).
 * No atomics: results are deterministic.
 * Accuracy: with fp16 inputs the recomputed exponent uses K (dK/dV) and Q
 * (dQ) multiplied by scale*log2(e) and rounded to fp16 (at most 2^-11
 * relative per element, the order of the rounding of P and dS that the
 * 16-bit matrix products need); bf16 inputs keep the scale in fp32.
 *
 *   q, k, v, o, lse : as produced for / by flash_attn_fwd (read)
 *   dout            : [B,H,N,d] gradient of O, of the input type (read)
 *   dq, dk, dv      : [B,H,N,d] of the input type (written)
 *   workspace       : device buffer of >= flash_attn_bwd_workspace_bytes(...)
 *                     bytes, 16-byte aligned, owned by the caller; its
 *                     contents on entry do not matter and on return are
 *                     unspecified.
 */
int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   void* stream);

/*
 * Backward of flash_attn_fwd_bias: the same gradients of L = <dO, O> with
 * P_ij = exp(scale * q_i . k_j + bias_ij - LSE_i) rebuilt from the bias and
 * the LSE flash_attn_fwd_bias wrote (the bias is a constant: its own
 * gradient, dS, is not formed).  Rows whose every key is hidden contribute
 * nothing.  Arguments as flash_attn_bwd, plus bias and its strides exactly as
 * passed to flash_attn_fwd_bias (same checks).
 */
int flash_attn_bwd_bias(const void* q, const void* k, const void* v, const void* bias,
                        long long bias_stride_b, long long bias_stride_h, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                        float scale, int causal, int dtype, void* stream);

/*
 * The three stages of flash_attn_bwd, callable on their own (same arguments,
 * layouts and checks as flash_attn_bwd; flash_attn_bwd is exactly these three
 * in order on one stream).  dK/dV and dQ only read the workspace the
 * preprocess wrote, so once it has run they may run on different streams.
 *
 * flash_attn_bwd_preprocess: -D_i (D_i = sum_c dO_ic O_ic, stored negated) and
 *   LSE_i*log2(e) into the workspace (page 2, "Re-computation": the per-row
 *   terms the recompute needs).
 *   `dtype` selects the input type and O's type as for the forward.
 * flash_attn_bwd_dkdv: dK and dV.  Each workgroup keeps a K/V tile and loops
 *   over query tiles, the loop order of that section.
 * flash_attn_bwd_dq: dQ.  Each workgroup keeps a query tile and loops over
 *   K/V tiles.
 */
int flash_attn_bwd_preprocess(const void* o, const float* lse, const void* dout,
                              void* workspace, size_t workspace_bytes,
                              int B, int H, int N, int d, int dtype, void* stream);
int flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                        const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                        int B, int H, int N, int d, float scale, int causal, int dtype,
                        void* stream);
int flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                      const void* workspace, size_t workspace_bytes, void* dq,
                      int B, int H, int N, int d, float scale, int causal, int dtype,
                      void* stream);

/*
 * Forward with an additive attention bias.  Page 2, "工程落地的关键考量",
 * suggests an attention bias to mask scores at very long sequences; this
 * adds one to every score before the softmax:
 *     O = softmax(scale * Q K^T + bias) V,
 *     LSE_i = ln sum_{j visible} exp(scale * q_i . k_j + bias_ij)
 * (-inf entries hide keys; the causal flag still applies on top).  A row
 * whose every score is -inf gets O = 0 and LSE = -inf.
 *
 *   bias          : input type (fp16 / bf16, as dtype), read-only.  For batch
 *                   b and head h the bias is the row-major N x N block at
 *                   element offset b*bias_stride_b + h*bias_stride_h (rows of N
 *                   elements, row i = query i, column j = key j); a stride of 0
 *                   broadcasts over that axis.  Entries are finite or -inf.
 *   bias_stride_b, bias_stride_h : element strides, >= 0 (FA_ERR_SHAPE),
 *                   multiples of 8 (FA_ERR_ALIGN)
 *   other arguments as flash_attn_fwd; in addition N must be a multiple of 8
 *   (16-byte bias rows; FA_ERR_ALIGN) and at most 46340 (one head's bias spans
 *   < 2^32 bytes; FA_ERR_SHAPE).
 */
int flash_attn_fwd_bias(const void* q, const void* k, const void* v, const void* bias,
                        long long bias_stride_b, long long bias_stride_h, void* o, float* lse,
                        int B, int H, int N, int d, float scale, int causal, int dtype,
                        void* stream);

/*
 * Split-KV forward.  The same result as flash_attn_fwd, computed as page 2's
 * "Tiling" pass cut along the key axis: the key tiles each query tile visits
 * are divided into num_splits contiguous ranges, each handled by its own
 * workgroup, which keeps the chip full when B*H*N is small (few query tiles)
 * or the keys are long.  Each range produces its own normalised O and LSE in
 * float32 (a range with no visible key for a row gives O = 0, LSE = -inf);
 * a second kernel merges them exactly:
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * (The online softmax's rescaling identity applied once per range instead of
 * once per tile.)
 *
 *   q, k, v, o, lse, B, H, N, d, scale, causal, dtype : as flash_attn_fwd
 *   workspace   : device buffer of >= flash_attn_fwd_splitkv_workspace_bytes
 *                 bytes, 16-byte aligned, owned by the caller; contents on
 *                 entry do not matter and on return are unspecified
 *   num_splits  : 1..64: every query tile's keys split that many ways
 *                 (splits beyond the number of key tiles are empty and cost
 *                 one idle workgroup each); 0: an automatic plan for this
 *                 shape, chosen by a cost model of whole rounds of concurrent
 *                 workgroups (two per compute unit, one at d=256): no split
 *                 (then it equals flash_attn_fwd and needs no workspace), a
 *                 uniform split, or (non-causal) a tail split, in which the
 *                 query tiles that fill whole rounds run unsplit and write O
 *                 directly and only the last, partial round's tiles are
 *                 split; other values give FA_ERR_SPLITS
 *   Up to three kernels are enqueued on `stream`.
 */
int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           void* workspace, size_t workspace_bytes,
                           int B, int H, int N, int d, float scale, int causal, int dtype,
                           int num_splits, void* stream);

/* Bytes of workspace flash_attn_fwd_splitkv needs: 4 * num_splits * B*H*N*(d+1)
 * (partial O and LSE); for num_splits = 0 what the automatic plan needs
 * (the larger of its causal and non-causal plans; 0 when it does not split);
 * 0 for invalid arguments. */
size_t flash_attn_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits);

/* A split count for this shape, in 1..16: more than 1 only when the unsplit
 * grid has at most one workgroup per compute unit and each split keeps at
 * least 32 key tiles (splitting adds a float32 partial O per split and a merge
 * pass, which shorter ranges do not repay). */
int flash_attn_fwd_splitkv_default_splits(int B, int H, int N, int d, int causal);

/* Bytes of workspace flash_attn_bwd needs (8 * B * H * N: two floats per row,
 * -D and -LSE*log2(e)); 0 for invalid sizes. */
size_t flash_attn_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Allocation-free backward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid allocation.  Same computation, kernels, arguments, checks and
 * results (bit for bit) as flash_attn_bwd, without the workspace arguments:
 * its -D and -LSE*log2(e) rows live in a static device array of
 * FA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on until the process ends (the address is looked up once per device,
 * on the first call with that device current).  The call itself allocates
 * nothing; the caller still provides every input and output.
 *   Limit: 8 * B * H * N <= FA_NOALLOC_SCRATCH_BYTES (B*H*N <= 2,097,152
 *   rows), else FA_ERR_SCRATCH before anything is launched.
 *   Concurrency: all calls on one device share that device's array, so calls
 *   whose work overlaps in time on one device (different streams, or host
 *   threads without ordering) race and give wrong gradients; calls ordered on
 *   one stream are safe.  Each call rewrites every row it reads, so nothing
 *   left by an earlier call is used.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int N, int d, float scale, int causal, int dtype,
                           void* stream);

/* Static, NUL-terminated description of a status code. */
const char* flash_attn_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int flash_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H_ */
