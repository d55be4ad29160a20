/*
 * fa_bwd.h -- C ABI of the MI355X (gfx950) FlashAttention-2 backward library
 * (libfa_bwd.so).
 *
 * The method: "CUDA 算子工程：手写 FlashAttention v2 之路", chapter 16 "FA2 反向：
 * dQ/dK/dV 的重计算".  Given Q, K, V, O, dO and the per-row logsumexp L of the
 * forward, the backward produces dQ, dK and dV without materialising the N x N
 * probability matrix: a preprocess computes D = rowsum(O * dO) (sec 16.1 and
 * sec 16.8 item 1), the main step runs key blocks outer and query blocks
 * inner (sec 16.2), recomputes S = scale * Q K^T and P = exp(S - L) on chip
 * (sec 16.4), forms dS = P * (dP - D) and accumulates dV = P^T dO, dK = dS^T Q
 * per key block, and dQ = dS K goes to an fp32 buffer (sec 16.3, the fp32
 * accumulation-buffer variant) -- summed by a second, query-outer pass rather
 * than by atomics (sec 16.3 weighs the two) -- and a convert step scales dQ and
 * casts it (sec 16.3 and 16.6).
 *
 * Conventions shared by every entry point
 *   Layout     Q, K, V, O, dO, dQ, dK, dV: contiguous [B, H, N, d] row-major
 *              (d fastest) in the element type `dtype`.  L, D: contiguous
 *              [B, H, N] fp32.  dq_accum: contiguous [B, H, N, d] fp32.
 *   dtype      FA_DTYPE_F32 (IEEE float), FA_DTYPE_BF16 (bfloat16 bits) or
 *              FA_DTYPE_F16 (IEEE half bits).  L, D and dq_accum are always
 *              fp32.  16-bit outputs are rounded to nearest even.  In fp16 the
 *              kernels hold P and dS as fp16 operands: inputs whose dS would
 *              exceed the half range (|dS| > 65504) are outside the contract.
 *   Scores     S_ij = scale * Q_i . K_j; L_i = log sum_j exp(S_ij) over the
 *              visible keys (natural log).  causal != 0 hides key j from
 *              query i when j > i (0-based, diagonal kept).  The softmax
 *              scale (1/sqrt(d) on the pages) must be finite and positive:
 *              the attention calls return FA_EINVAL otherwise (the
 *              convert step only multiplies by it and takes any value).
 *   Pointers   device pointers (hipMalloc'd or equivalent), owned by the
 *              caller, at least 16-byte aligned, each to a buffer holding at
 *              least the elements its layout implies for the call's B, H, N
 *              and d (the library cannot check this: a smaller buffer is read
 *              or written out of bounds).  Outputs must not alias inputs.
 *              The library allocates nothing; its only mutable global state
 *              is fa_bwd_noalloc's static scratch array (see there) and
 *              device properties it queries once and keeps (each device's CU
 *              count, the kernels' resident workgroups per CU).  Calls on
 *              different streams may run concurrently as long as their
 *              buffers are disjoint (fa_bwd_noalloc calls excepted).
 *   Stream     `stream` is a hipStream_t passed as void*; NULL is the null
 *              stream.  Every call only enqueues work and returns; the caller
 *              synchronises.  No call allocates, clears memory with a memset
 *              or synchronises, so calls can be captured into a HIP graph
 *              (after one eager call on the device, which makes the one-time
 *              queries).
 *   Sizes      B, H, N, d >= 1; B * H * N * d < 2^40; B and H < 65536;
 *              N <= 2^30 (row and tile indices are 32-bit).
 *              Supported head dims: d in {16, 32, 64, 128} for every dtype.
 *   Errors     every call returns an fa_status_t.  Arguments are validated
 *              before any device work: FA_EINVAL for a NULL pointer, a
 *              non-positive or oversized dimension, an unknown dtype or a
 *              softmax scale that is not finite and positive;
 *              FA_EUNSUPPORTED for an unsupported head dim.  FA_EHIP when the
 *              HIP runtime reports an error (no device, launch failure); the
 *              raw hipError_t is available from fa_last_hip_error().  No call
 *              aborts or throws.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_DTYPE_F32 = 0, FA_DTYPE_BF16 = 1, FA_DTYPE_F16 = 2 } fa_dtype_t;

typedef enum {
    FA_OK = 0,
    FA_EINVAL = 1,
    FA_EUNSUPPORTED = 2,
    FA_EHIP = 3,
    FA_ESCRATCH = 4  /* fa_bwd_noalloc only: B * H * N above FA_NOALLOC_MAX_ROWS */
} fa_status_t;

/* Rows (B * H * N) that fa_bwd_noalloc's static scratch array holds: 16 MiB of
 * fp32 per GPU. */
#define FA_NOALLOC_MAX_ROWS (1 << 22)

/*
 * fa_fwd_lse -- attention forward producing O and the logsumexp L that the
 * backward consumes.  Query blocks outer, key blocks inner with the online
 * softmax (running max m, denominator l, accumulator a rebased by
 * alpha = exp(m - m') at each key block), O = a / l and L = m + log l
 * (1point3acres post "手扒了FlashAttention", the online-softmax recurrence and
 * the logsumexp; FA2 chapter 16 sec 16.4).  Supporting step of the backward:
 * it provides O and L for benchmarking and end-to-end checks.  bf16 and fp16
 * with d = 64 or 128 run on the matrix cores and rebase lazily (only when a block's
 * maximum exceeds the running one by more than a factor 2^8, which leaves
 * O and L unchanged in exact arithmetic); other cases run a vector-ALU kernel.
 *   in : Q, K, V [B,H,N,d] dtype
 *   out: O [B,H,N,d] dtype (rounded to nearest even for bf16), L [B,H,N] fp32
 */
int fa_fwd_lse(int dtype, const void* Q, const void* K, const void* V,
               void* O, float* L,
               int B, int H, int N, int d, float scale, int causal,
               void* stream);

/*
 * fa_lse -- the logsumexp L alone, for a backward whose forward did not store
 * it.  FA2 chapter 16 sec 16.4 names the cost: the online softmax has to run
 * once more, a full sweep over K (the chapter's closing exercise asks for
 * it).  The same query-outer sweep as fa_fwd_lse with V and O left out: the
 * running maximum m and denominator l per row, L = m + log l (natural log),
 * bitwise the same L as fa_fwd_lse on the same inputs.
 *   in : Q, K [B,H,N,d] dtype
 *   out: L [B,H,N] fp32
 */
int fa_lse(int dtype, const void* Q, const void* K, float* L,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_bwd_preprocess -- D_i = sum_k O_ik dO_ik with fp32 accumulation (FA2
 * chapter 16 sec 16.1, the identity D_i = dO_i . O_i, and sec 16.8 item 1:
 * computed once before the main loop).  dq_accum needs no clearing (fa_bwd
 * writes every element of it), so this step touches D only.
 *   in : O, dO [B,H,N,d] dtype
 *   out: D [B,H,N] fp32 (every element written)
 */
int fa_bwd_preprocess(int dtype, const void* O, const void* dO, float* D,
                      int B, int H, int N, int d, void* stream);

/*
 * fa_bwd -- the main backward step (FA2 chapter 16 sec 16.2 loop order, sec
 * 16.6 skeleton): it recomputes S = scale Q K^T and P = exp(S - L), forms
 * dP = dO V^T and dS = P (dP - D), and accumulates dV = P^T dO and dK = dS^T Q
 * per key block (dK multiplied by `scale` at write-out, sec 16.6) and
 * dQ = dS K (unscaled) per query block; under the causal mask, tiles wholly
 * above the diagonal are skipped (sec 16.8 item 2).  It runs both passes in
 * one launch, and its results are bitwise those of fa_bwd_dq followed by
 * fa_bwd_dkdv on the same stream.
 *   One contract for every dtype and head dim: dq_accum is overwritten (its
 *   prior contents are never read), no atomics are used, and dq_accum, dK
 *   and dV are bitwise reproducible from call to call.  bf16 and fp16 with
 *   d = 64 or 128 run on the matrix cores; fp32, and 16-bit d = 16 or 32, on
 *   the vector ALUs.
 *   in : Q, K, V, dO [B,H,N,d] dtype; L, D [B,H,N] fp32
 *   out: dq_accum [B,H,N,d] fp32 = sum_j dS_ij K_j (unscaled);
 *        dK, dV [B,H,N,d] dtype
 */
int fa_bwd(int dtype, const void* Q, const void* K, const void* V,
           const void* dO, const float* L, const float* D,
           float* dq_accum, void* dK, void* dV,
           int B, int H, int N, int d, float scale, int causal,
           void* stream);

/*
 * fa_bwd_dkdv / fa_bwd_dq -- the two passes fa_bwd runs, callable on their
 * own (same arguments and layouts as fa_bwd, every dtype and head dim).  FA2
 * chapter 16 sec 16.3 weighs fp32 global atomics for dQ against a second
 * kernel; on MI355X the atomics measured too slow (about 340 G fp32
 * atomics/s), so dQ has its own query-outer pass:
 *   fa_bwd_dkdv: key blocks outer, query tiles inner (sec 16.2); recomputes S,
 *                P, dP, dS and accumulates dV = P^T dO, dK = scale dS^T Q.
 *   fa_bwd_dq:   query blocks outer, key blocks inner; recomputes S, P, dP, dS
 *                and accumulates dQ = dS K, written once (unscaled) into
 *                dq_accum -- no atomics, bitwise reproducible.
 */
int fa_bwd_dkdv(int dtype, const void* Q, const void* K, const void* V,
                const void* dO, const float* L, const float* D,
                void* dK, void* dV,
                int B, int H, int N, int d, float scale, int causal,
                void* stream);
int fa_bwd_dq(int dtype, const void* Q, const void* K, const void* V,
              const void* dO, const float* L, const float* D, float* dq_accum,
              int B, int H, int N, int d, float scale, int causal,
              void* stream);

/*
 * fa_bwd_convert_dq -- dQ = scale * dq_accum cast to dtype (round to nearest
 * even for bf16 and fp16) (FA2 chapter 16 sec 16.3: the separate kernel that applies
 * the softmax scale and converts the fp32 accumulation buffer).
 *   in : dq_accum [B,H,N,d] fp32
 *   out: dQ [B,H,N,d] dtype
 */
int fa_bwd_convert_dq(int dtype, const float* dq_accum, void* dQ,
                      int B, int H, int N, int d, float scale, void* stream);

/*
 * fa_bwd_noalloc -- the whole backward (fa_bwd_preprocess, fa_bwd and
 * fa_bwd_convert_dq in one call) without any device allocation and without a
 * caller workspace, for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *   D lives in a static device array of the library (FA_NOALLOC_MAX_ROWS fp32,
 *   one per GPU, kept until the process ends; its address is looked up on the
 *   first call on each device); dq_accum is not needed: the dQ pass writes
 *   dQ = scale * (sum_j dS_ij K_j) in the element type itself, the same values
 *   fa_bwd_convert_dq makes of dq_accum.  Outputs equal those of the three
 *   calls bit for bit.
 *   Calls of one process that overlap on one GPU (concurrent streams or
 *   threads) race on that GPU's scratch array: serialise them.  Sequential
 *   calls on one stream are safe; every call rewrites the D rows it reads.
 *   in : Q, K, V, O, dO [B,H,N,d] dtype; L [B,H,N] fp32
 *   out: dQ, dK, dV [B,H,N,d] dtype
 *   errors: as fa_bwd; FA_ESCRATCH when B * H * N > FA_NOALLOC_MAX_ROWS.
 */
int fa_bwd_noalloc(int dtype, const void* Q, const void* K, const void* V,
                   const void* O, const void* dO, const float* L,
                   void* dQ, void* dK, void* dV,
                   int B, int H, int N, int d, float scale, int causal,
                   void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(int status);

/* The hipError_t of the calling thread's most recent FA_EHIP, or 0. */
int fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
