/*
 * fa.h -- C ABI of libfa.so: exact tiled attention (FlashAttention forward and
 * backward) on AMD Instinct MI355X (gfx950).
 *
 * The operation is softmax attention per (batch, head):
 *
 *   S = scale * Q K^T,  P = softmax(S) row-wise,  O = P V,
 *   L_i = logsumexp_j S_ij  (natural log),
 *
 * computed tile by tile with an online softmax so that S and P never reach
 * HBM; only O and the per-row logsumexp L are written.  The interface and
 * outputs follow the "FlashAttention" deep-dive page (tirogla.com), section
 * "How it works": per head the caller supplies N x d matrices Q, K, V and
 * receives O plus one logsumexp value per query row; no state is kept
 * between calls.  The backward recomputes P from
 * L and forms dQ, dK, dV from D = rowsum(dO * O) and dS = P * (dP - D) (same
 * section).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers into memory the caller owns.  The
 *    library allocates nothing, keeps no state between calls and may be called
 *    concurrently on different streams.
 *  - Layout: row-major contiguous [B, H, N, d] for q, k, v, o, dO, dq, dk, dv;
 *    [B, H, N] for lse and delta.  Base pointers must be 16-byte aligned.
 *    Outputs must not alias inputs.
 *  - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16);
 *    bf16 outputs are rounded to nearest, ties to even.
 *  - causal != 0 applies the square, top-left aligned mask: key j is visible to
 *    query i iff j <= i.  Tiles entirely above the diagonal are skipped.
 *  - scale is any finite float, positive, negative or zero, with
 *    |scale| * log2(e) finite in fp32; callers usually pass 1/sqrt(d).  (The
 *    kernels fold the sign, or a zero, into one operand of S exactly, so the
 *    scores are bitwise scale times the fp32 sum of products.)  The scaled
 *    scores themselves must stay inside the fp32 range.
 *  - lse is the natural-log logsumexp of the SCALED scores (the value that the
 *    deep-dive page's pseudocode stores as L = m + log l).
 *  - Calls are asynchronous on `stream` (0 = the null stream); outputs are
 *    valid once the stream reaches the call.  The host never synchronises.
 *  - Arguments are validated before any launch; on an error nothing is
 *    launched and outputs are untouched.  No exception crosses the ABI.
 *
 * Supported shapes: B, H, N >= 1 with B*H <= 2^31-1, B*H*N*d < 2^62 (element
 * offsets are 64-bit), N*d*4 < 2^31 (one head is addressed through a 32-bit
 * buffer range: N <= 4194303 at d = 128), d in {64, 128}.
 * Inputs must be finite: the kernels are built without IEEE NaN handling, so
 * NaN or infinite inputs give unspecified outputs.
 */
#ifndef FA_H
#define FA_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* null pointer, B/H/N < 1, Hkv not dividing Hq, scale not finite (or
                               |scale| log2(e) overflowing fp32), size overflow, decode workspace too small */
    FA_ERR_UNSUPPORTED = 2, /* head dimension d not in {64, 128} */
    FA_ERR_HIP = 3,         /* the HIP runtime reported an error at launch */
    FA_ERR_SCRATCH = 4      /* fa_bwd_noalloc: B*H*N exceeds FA_NOALLOC_MAX_ROWS */
} fa_status;

/*
 * Forward, bf16 inputs and output, fp32 arithmetic.
 *   q, k, v : const bf16 [B,H,N,d]
 *   o       : bf16 [B,H,N,d]      attention output, O = softmax(scale Q K^T) V
 *   lse     : float [B,H,N]       natural-log logsumexp of each scaled score row
 * S, the running row max/sum and the output accumulator are fp32; P is rounded
 * to bf16 only as the operand of the P V product (deep-dive page,
 * "Implementation notes").
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Forward, fp32 inputs and output.  Same semantics as fa_fwd; every product
 * and sum is fp32 (P is not rounded to bf16).
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Attention dropout ("FlashAttention" deep-dive page, "Implementation notes":
 * the mask is never written out; the backward draws it again from a Philox
 * seed and offset).  As fa_fwd_gqa / fa_bwd_gqa, with each attention probability
 * P_ij of flat query head bh = b*Hq + h dropped with probability thr/256 and
 * kept ones scaled by 256/(256 - thr), thr = min(255, floor(256 dropout_p + 1/2)):
 *   O = (P * Z) V,  Z_ij = keep_ij * 256/(256 - thr);  lse is that of the
 *   undropped scores;  the backward uses the same Z (dS = P (Z dP - D)).
 * keep_ij: byte 8 (j%4) of word (j/8)%4 of Philox4x32-10 (Salmon et al., SC
 * 2011) with counter (2 (j/32) + (j/4)%2, i, bh, offset) and key (seed low
 * 32 bits, seed high 32 bits) is >= thr.  Calls with the same seed and offset
 * draw the same mask; fa_bwd_dropout must be given the forward's.
 *   dropout_p : in [0, 1);  offset : below 2^32.
 * Errors as for fa_fwd_gqa / fa_bwd_gqa, plus FA_ERR_INVALID_ARG for
 * dropout_p outside [0, 1) or offset >= 2^32.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                   float dropout_p, unsigned long long seed, unsigned long long offset, hipStream_t stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, float* dq, float* dk, float* dv, float* delta,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                   float dropout_p, unsigned long long seed, unsigned long long offset, hipStream_t stream);

/*
 * Forward with fp8 inputs (the low-precision forward the deep-dive pages name
 * for FlashAttention-3: "FlashAttention" deep-dive page, "Implementation
 * notes"; "Why Flash Attention Is Fast", FlashAttention-3 section).
 *   q, k, v : const fp8 [B,Hq,N,d] / [B,Hkv,N,d] / [B,Hkv,N,d], OCP e4m3 bytes
 *             (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 *             infinities; 0x7F and 0xFF are NaN and must not occur)
 *   q_descale, k_descale, v_descale : finite, > 0; the real inputs are
 *             q_descale * q, k_descale * k, v_descale * v
 *   o       : bf16 [B,Hq,N,d]   O = softmax(scale (q_descale q)(k_descale k)^T) (v_descale v)
 *   lse     : float [B,Hq,N]    natural-log logsumexp of the scaled scores
 * S is accumulated in fp32 from exact fp8 products; P is computed in fp32 and
 * rounded to e4m3 only as the operand of the P V product, while the row sum
 * l is taken over the unrounded P.  Grouped heads as for fa_fwd_gqa (Hkv = Hq
 * for one key/value head per query head).  Errors as for fa_fwd_gqa, plus
 * FA_ERR_INVALID_ARG for a factor that is not finite and positive.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, float scale,
               float q_descale, float k_descale, float v_descale, int causal, hipStream_t stream);

/*
 * Backward, bf16 inputs, fp32 gradients.
 *   q, k, v : const bf16 [B,H,N,d]  the forward's inputs
 *   o       : const bf16 [B,H,N,d]  the forward's output
 *   lse     : const float [B,H,N]   the forward's logsumexp (natural log)
 *   dO      : const bf16 [B,H,N,d]  gradient of the loss with respect to o
 *   dq, dk, dv : float [B,H,N,d]    gradients with respect to q, k, v (written,
 *                                   not accumulated into)
 *   delta   : float [B,H,N]         caller-provided workspace; receives
 *                                   D_i = sum_t dO_it * O_it
 * P is recomputed tile by tile as exp(scale q_i.k_j - L_i); dS = P * (dP - D);
 * dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.  dQ is accumulated by one
 * workgroup per query block (no atomics), so results are bitwise reproducible.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, float* dq, float* dk, float* dv, float* delta,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Grouped heads (GQA; MQA when Hkv = 1): several query heads share one key
 * and value head ("FlashAttention" deep-dive page, "Implementation notes":
 * the query head maps to its key/value head).  Per batch there are Hq query
 * heads and Hkv key/value heads, Hkv >= 1 dividing Hq; query head h of batch b
 * attends with key/value head h / (Hq / Hkv) of batch b.
 *
 * fa_fwd_gqa: as fa_fwd with
 *   q, o    : bf16 [B,Hq,N,d],   lse : float [B,Hq,N]
 *   k, v    : bf16 [B,Hkv,N,d]
 * fa_bwd_gqa: as fa_bwd with q, o, dO, dq [B,Hq,N,d], lse, delta [B,Hq,N] and
 *   k, v, dk, dv [B,Hkv,N,d]; dk and dv are the sums of the gradients of the
 *   Hq / Hkv query heads that share each key/value head (written, not
 *   accumulated into; still bitwise reproducible).
 * fa_fwd and fa_bwd are these with Hkv = Hq.  Errors as for fa_fwd/fa_bwd, plus
 * FA_ERR_INVALID_ARG when Hkv < 1 or Hq % Hkv != 0.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal, hipStream_t stream);
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dO, float* dq, float* dk, float* dv, float* delta,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_bwd_gqa with bf16 gradients: dq, dk, dv are bf16 (round to nearest even
 * of the fp32 accumulators) instead of fp32; everything else as fa_bwd_gqa.
 * Halves the gradients' HBM writes for callers that keep gradients in bf16.
 */
int fa_bwd_gqa_bf16grad(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, void* dk, void* dv, float* delta,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Split-KV decode (Flash-Decoding): one query row per (batch, query head)
 * against a key/value cache ("FlashAttention" deep-dive page, "Implementation
 * notes": with a single query row, chunks of the cache are processed in
 * parallel and their partial (m, l, acc) triples are merged with the same
 * rescaling rule).  Grouped heads as for fa_fwd_gqa (Hkv = Hq: one key/value
 * head per query head).
 *   q       : const bf16 [B,Hq,d]        the new token's query rows
 *   k, v    : const bf16 [B,Hkv,Nk,d]    the cache (Nk rows of capacity)
 *   kv_len  : const int [B] DEVICE pointer, or NULL: batch b attends to cache
 *             rows 0 .. kv_len[b]-1 (all Nk when NULL).  Values are clamped to
 *             [0, Nk] on the device; kv_len[b] = 0 gives O = 0, L = -inf.
 *   o       : bf16 [B,Hq,d]              O = softmax(scale q K^T) V per row
 *   lse     : float [B,Hq]               natural-log logsumexp of the scaled scores
 *   num_splits : chunks the cache is cut into; 0 lets the library choose.  The
 *             effective count (at most ceil(Nk / 256), chunks of a multiple of
 *             256 keys) is what fa_decode_plan reports.
 *   workspace, workspace_bytes : device memory for the partial triples, at
 *             least the size fa_decode_plan reports (0 bytes, and workspace may
 *             be NULL, when the effective split count is 1).  Overwritten.
 * The result depends on the split count only through rounding; for a fixed
 * count it is bitwise reproducible.  Errors as for fa_fwd_gqa, plus
 * FA_ERR_INVALID_ARG for Nk < 1, num_splits < 0, or a workspace that is NULL
 * or smaller than required.
 *
 * fa_decode_plan validates the same shape arguments and reports the effective
 * split count (*splits, may be NULL) and the workspace size in bytes
 * (*workspace_bytes, may be NULL) for num_splits.  It launches nothing.
 */
int fa_decode_plan(int B, int Hq, int Hkv, int Nk, int d, int num_splits, int* splits, size_t* workspace_bytes);
int fa_decode(const void* q, const void* k, const void* v, const int* kv_len, void* o, float* lse,
              int B, int Hq, int Hkv, int Nk, int d, float scale, int num_splits, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/*
 * The stages of fa_bwd, for callers that schedule or time them separately.
 * fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq in this order on one stream are
 * exactly fa_bwd (the kernels fa_bwd runs).  fa_bwd_dv and fa_bwd_dk compute
 * the same dV and dK as fa_bwd_dkdv, bitwise, with one kernel each (S is then
 * computed twice).
 *
 * fa_bwd_preprocess: delta[i] = sum_t dO_it * O_it (fp32), o and dO bf16.
 * fa_bwd_dkdv:       dK and dV (fp32) from q, k, v, dO (bf16), lse and delta.
 * fa_bwd_dv:         dV (fp32) from q, k, dO (bf16) and lse.
 * fa_bwd_dk:         dK (fp32) from q, k, v, dO (bf16), lse and delta.
 * fa_bwd_dq:         dQ (fp32) from q, k, v, dO (bf16), lse and delta.
 * Arguments have the meaning, layout and checks of fa_bwd.
 */
int fa_bwd_preprocess(const void* o, const void* dO, float* delta, int B, int H, int N, int d,
                      hipStream_t stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                const float* delta, float* dk, float* dv, int B, int H, int N, int d, float scale,
                int causal, hipStream_t stream);
int fa_bwd_dv(const void* q, const void* k, const float* lse, const void* dO, float* dv,
              int B, int H, int N, int d, float scale, int causal, hipStream_t stream);
int fa_bwd_dk(const void* q, const void* k, const void* v, const float* lse, const void* dO,
              const float* delta, float* dk, int B, int H, int N, int d, float scale, int causal,
              hipStream_t stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO,
              const float* delta, float* dq, int B, int H, int N, int d, float scale, int causal,
              hipStream_t stream);

/*
 * fa_bwd without the delta workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  The library keeps D = rowsum(dO * O)
 * in a static device array of FA_NOALLOC_MAX_ROWS floats (16 MiB), one per
 * GPU it runs on, held until the process ends; the call allocates nothing and
 * calls no allocating routine.  Every other argument, and the results
 * (bitwise those of fa_bwd), are as for fa_bwd.
 *   Limit: B*H*N <= FA_NOALLOC_MAX_ROWS, else FA_ERR_SCRATCH before any launch.
 *   The array of the CURRENT device (hipGetDevice) is used: `stream` must
 *   belong to that device.  The first call on a device looks the array's
 *   address up (hipGetSymbolAddress); a failure there returns FA_ERR_HIP.
 *   Calls that overlap on one GPU (other streams, other host threads) share
 *   the array and race: serialise them, e.g. on one stream.
 */
#define FA_NOALLOC_MAX_ROWS (1 << 22)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, float* dq, float* dk, float* dv,
                   int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
