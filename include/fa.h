/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library libfa.so.
 *
 * The library computes exact attention, O = softmax(scale * Q K^T) V, the
 * attention equation of "FlashAttention (DE)", section "Problematik der
 * Standard-Attention", as one fused, tiled kernel that streams K/V blocks
 * through on-chip memory and keeps a running row maximum and exponential sum
 * (sections "Tiling und blockweise Verarbeitung", "Online-Softmax-Berechnung",
 * "Zusammenfassen von Operationen in einem CUDA-Kernel").  The N x N score
 * matrix is never written to device memory.  The forward also returns the
 * per-row log-sum-exp; the backward keeps nothing else from the forward and
 * recomputes the score blocks from it (Dutch glossary page "FlashAttention",
 * section "Hoe werkt het?", bullet "Herberekening").
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates device memory and keeps no pointer after a call returns.
 *  - Tensors are contiguous row-major [B, H, N, d] (q, k, v, o, dout, dq, dk,
 *    dv) and [B, H, N] (lse).  The element type of q, k, v, o, dout, dq, dk,
 *    dv is `dtype`; lse is always float32.  Indexing is 64-bit.
 *  - Every tensor pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work; completion is observed by synchronising that
 *    stream.  Inputs are read-only; outputs are fully overwritten.  Outputs
 *    that overlap inputs or each other are undefined behaviour.
 *  - All arguments are validated before any HIP call.  On a validation error
 *    the status is returned and nothing is enqueued.  A failed launch maps to
 *    FA_ERR_HIP.  Nothing is printed; no exception crosses the ABI; the
 *    library holds no mutable global state, so calls are thread-safe.
 *  - causal = 1 applies the causal mask: query i sees key j iff j <= i
 *    (positions counted from 0; queries and keys have the same length N;
 *    fa_decode places its queries at the end of each cache, see there).
 *    Masked scores get probability exactly 0.
 *  - scale must be finite and > 0 (the pages' value is 1/sqrt(d)).
 *  - Supported: d in {64, 128}, and d in {32, 96, 256} in bf16 (fa_fwd, fa_bwd
 *    and their _gqa forms); fa_fwd_fp8 takes d in {64, 128, 256}; the fp32
 *    forward and fa_decode return FA_ERR_UNSUPPORTED_HEAD_DIM for other d;
 *    B, H, N >= 1; B*H*N*d < 2^62; one head's N*d elements below 2^31 bytes
 *    (N < 8,388,608 for bf16 at d = 128).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#if defined(__GNUC__)
#define FA_API __attribute__((visibility("default")))
#else
#define FA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_DTYPE_F32 = 0,  /* IEEE float32 inputs and outputs */
  FA_DTYPE_BF16 = 1  /* bfloat16 inputs and outputs, float32 accumulation */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1,         /* a required pointer is NULL */
  FA_ERR_BAD_SHAPE = 2,            /* B, H or N < 1, the element count overflows, or Hq % Hkv != 0 */
  FA_ERR_UNSUPPORTED_HEAD_DIM = 3, /* d not supported by this entry point (see "Supported" above) */
  FA_ERR_UNSUPPORTED_DTYPE = 4,    /* dtype unknown, or not supported by this entry point */
  FA_ERR_BAD_SCALE = 5,            /* scale not finite or not > 0 */
  FA_ERR_MISALIGNED = 6,           /* a tensor pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE_TOO_SMALL = 7,  /* workspace NULL or smaller than fa_bwd_workspace_size() */
  FA_ERR_HIP = 8,                  /* a HIP launch or runtime call failed */
  FA_ERR_BAD_ARGUMENT = 9,         /* causal not 0 or 1 (appended after the original eight codes) */
  FA_ERR_SCRATCH_TOO_SMALL = 10    /* fa_bwd_noalloc: the problem needs more than the static scratch */
} fa_status_t;

/*
 * Forward: o = softmax(scale * q k^T [causal mask]) v and, per query row,
 * lse = ln sum_j exp(scale * q_i . k_j) over the visible keys (natural log,
 * float32).  The lse is the normalisation value that fa_bwd consumes.
 *
 *   q, k, v : [B,H,N,d] inputs of `dtype`.
 *   o       : [B,H,N,d] output of `dtype`.
 *   lse     : [B,H,N] float32 output.
 * dtype FA_DTYPE_BF16 runs both products on bf16 matrix cores with float32
 * accumulation (P is rounded to bf16, nearest-even, before multiplying V);
 * FA_DTYPE_F32 computes in float32 throughout.  No workspace: the forward
 * uses no device memory beyond its arguments.
 */
FA_API int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, int causal, float scale, int dtype,
           void *stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: per query row,
 * D_i = sum_c dO_ic O_ic and lse_i * log2(e), float32 [2][B,H,N], rounded up
 * to 256 bytes.  Returns 0 for arguments fa_bwd would reject.
 */
FA_API size_t fa_bwd_workspace_size(int B, int H, int N, int d, int dtype);

/*
 * Backward with recomputation.  Given the forward's inputs, its output o and
 * its lse, and the upstream gradient dout = dL/dO, writes dq, dk, dv.  The
 * score and probability blocks are recomputed from q, k and lse; nothing of
 * size N x N is stored.
 *
 *   q, k, v, o, dout : [B,H,N,d] inputs of `dtype`.
 *   lse              : [B,H,N] float32 from fa_fwd on the same q, k, v.
 *   dq, dk, dv       : [B,H,N,d] outputs of `dtype`.
 *   workspace        : device memory of at least fa_bwd_workspace_size()
 *                      bytes, 16-byte aligned; contents on entry are ignored
 *                      and are garbage on exit.
 * Only FA_DTYPE_BF16 is supported (FA_ERR_UNSUPPORTED_DTYPE otherwise).
 * Two kernels run on `stream`: one owns a block of queries and produces dq
 * (and the per-row D and scaled lse in the workspace), the other owns a block
 * of keys and produces dk and dv (at d = 256 two launches of it, one for dv
 * and one for dk, since one wave cannot hold both accumulators).  No atomics
 * are used, so dq, dk and dv are bitwise reproducible.
 */
FA_API int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const void *dout, const float *lse, void *dq, void *dk, void *dv,
           void *workspace, size_t workspace_bytes,
           int B, int H, int N, int d, int causal, float scale, int dtype,
           void *stream);

/*
 * fa_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results as fa_bwd, without the workspace arguments:
 * the per-row workspace lives in a static device array of the library
 * (fa_bwd_noalloc_scratch_bytes() = 16 MiB, which covers B*H*N up to 2^21
 * query rows, e.g. B=1 H=32 N=65536).  Larger problems return
 * FA_ERR_SCRATCH_TOO_SMALL and enqueue nothing.  The call allocates nothing
 * (no hipMalloc, no library allocation); its first call on a device looks up
 * that device's copy of the array once (hipGetSymbolAddress), and each device
 * keeps its copy until the process ends.  The array is shared by every call on
 * a device: calls that overlap on one device (on different streams, or from
 * different threads without ordering) race and give undefined results.  The
 * backward needs no part of it zeroed.  The current device must be the one
 * that owns the tensors and the stream.
 */
FA_API int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                   const void *dout, const float *lse, void *dq, void *dk, void *dv,
                   int B, int H, int N, int d, int causal, float scale, int dtype,
                   void *stream);
FA_API size_t fa_bwd_noalloc_scratch_bytes(void);

/*
 * Query heads sharing key/value heads (multi-query attention, which
 * "FlashAttention (DE)", section "Evolution und Weiterentwicklungen", lists
 * among the FlashAttention-2 capabilities, and its grouped generalisation).
 * There are Hq query heads and Hkv key/value heads, Hkv >= 1 dividing Hq;
 * query head h attends with K/V head h / (Hq / Hkv) (contiguous groups).
 * Hkv = 1 is multi-query attention; Hkv = Hq is exactly fa_fwd / fa_bwd, which
 * are these calls with Hq = Hkv = H.
 *
 *   q, o, dout, dq : [B,Hq,N,d];  k, v, dk, dv : [B,Hkv,N,d];  lse : [B,Hq,N].
 *
 * The gradient of a shared K/V head is the sum over its query heads; the
 * kernel that owns a block of keys runs over the query heads of the group.
 * When B*Hkv*ceil(N/128) key blocks are too few to fill the GPU, the group's
 * query heads are split over S = min(Hq/Hkv, ceil(512 / (B*Hkv*ceil(N/128))))
 * workgroups per key block, each writing float32 partial dk and dv into the
 * workspace, and a third kernel sums the S partials in a fixed order.  No
 * atomics are used, so dq, dk and dv are bitwise reproducible.
 * fa_bwd_gqa_workspace_size = 2*B*Hq*N*4 bytes rounded up to 256, plus
 * 2*S*B*Hkv*N*d*4 bytes when S > 1.  Hkv < 1 or Hq not a multiple of Hkv gives
 * FA_ERR_BAD_SHAPE.  Everything else is as for fa_fwd / fa_bwd_workspace_size
 * / fa_bwd.
 */
FA_API int fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               int dtype, void *stream);
FA_API size_t fa_bwd_gqa_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype);
FA_API int fa_bwd_gqa(const void *q, const void *k, const void *v, const void *o,
               const void *dout, const float *lse, void *dq, void *dk, void *dv,
               void *workspace, size_t workspace_bytes,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               int dtype, void *stream);

/*
 * Attention of a few new query rows against a key/value cache (decode), the
 * serving case "FlashAttention (DE)", section "Evolution und
 * Weiterentwicklungen", subsection "Spezialisierte Lösungen" names
 * (FlashInfer: the KV cache in streaming generation).
 *
 *   q       : [B,Hq,Nq,d] bf16, the Nq newest positions of each sequence.
 *   k, v    : [B,Hkv,Nk,d] bf16 cache; Nk is its capacity.  Query heads share
 *             K/V heads as in fa_fwd_gqa (Hkv divides Hq).
 *   kv_lens : device int32 [B], the valid cache rows L_b of each sequence, or
 *             NULL for L_b = Nk.  Values are clamped to [0, Nk].
 *   o       : [B,Hq,Nq,d] bf16 output;  lse : [B,Hq,Nq] float32 output.
 * Query i of sequence b sits at position L_b - Nq + i.  It attends to cache
 * rows j < L_b; with causal = 1 only to j <= L_b - Nq + i.  A query that sees
 * no row gets o = 0 and lse = -inf.
 * Cache rows j >= L_b are never read (they may hold anything, NaN included).
 * Only FA_DTYPE_BF16 and d in {64, 128}.  The workspace (at least
 * fa_decode_workspace_size() bytes, 16-byte aligned; its contents on entry do
 * not matter) holds float32 partial results: the key tiles of all sequences
 * and K/V heads are divided evenly over one wave per SIMD of the GPU so that K
 * and V stream from HBM once at full bandwidth, and a second kernel merges the
 * partial results (lse = ln sum_p e^lse_p, o = sum_p e^(lse_p - lse) o_p).
 * The size depends on B, Hq, Hkv, Nq and d only (at most 2048 waves).  Results
 * are bitwise reproducible on a given GPU model (the division over waves
 * follows its compute-unit count).
 * fa_decode_workspace_size returns 0 for arguments fa_decode would reject.
 */
FA_API size_t fa_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int dtype);
FA_API int fa_decode(const void *q, const void *k, const void *v, const int *kv_lens,
              void *o, float *lse, void *workspace, size_t workspace_bytes,
              int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
              int dtype, void *stream);

/*
 * Forward with FP8 inputs, the low-precision mode of FlashAttention-3
 * ("FlashAttention (DE)", section "Evolution und Weiterentwicklungen",
 * subsection "FlashAttention-3 (2024)").
 *
 *   q : [B,Hq,N,d], k, v : [B,Hkv,N,d]  one byte per element, OCP FP8 E4M3
 *       codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 *       infinities; 0x7F / 0xFF are NaN).  Each tensor carries one float32
 *       scale: the value of code c is e4m3(c) * x_scale.
 *   o   : [B,Hq,N,d] bf16 output;  lse : [B,Hq,N] float32 output (natural log
 *         of the row sum of exp(scale * s_ij), s_ij the scaled-input scores).
 * Query heads share K/V heads as in fa_fwd_gqa.  Both products run on the
 * FP8 matrix cores with float32 accumulation.  The probabilities of each key
 * block are rounded to E4M3 before they multiply V (relative error up to
 * 2^-4 each, one extra subnormal step below 2^-6 of the running row maximum),
 * and the row sum is taken over the same rounded values, so o is a convex
 * combination of rows of V with weights within that rounding of the exact
 * ones.  q_scale, k_scale, v_scale must be finite and > 0, and
 * q_scale * k_scale * scale must stay a normal float (FA_ERR_BAD_SCALE).
 * d in {64, 128, 256}.  Everything else is as for fa_fwd_gqa.
 */
FA_API int fa_fwd_fp8(const void *q, const void *k, const void *v,
               float q_scale, float k_scale, float v_scale, void *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               void *stream);

/* A static, human-readable string for a status code (never NULL). */
FA_API const char *fa_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
FA_API int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
