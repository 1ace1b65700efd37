/*
 * li.h -- C ABI of the MI355X (gfx950) lightning-indexer library (liblightning_indexer.so).
 *
 * The library implements the key-selection hot path of natively sparse attention:
 *
 *   1. indexer scoring: every visible compressed key s of a query row is scored as
 *        score(s) = sum_h w[h] * max(q[h] . k[s], 0)
 *      ("Long context", llm-serving.xyz lecture 03, section "The Architectural
 *      Answer: Read Less of the Past", paragraph "Stage 1, the lightning indexer":
 *      one 128-d FP8 key per position, shared by all indexer heads, 128 B + a 4 B
 *      scale; the output is only a ranking);
 *   2. top-k selection of the best k keys per row (same page, paragraph "Stage 2,
 *      sparse main attention"; LeanSparse podcast transcript, cue 01:33, k = 512;
 *      "Latent Sparse Attention" article, section "What the kernels do about the
 *      top-p": packed keys with the score above an inverted id, engine cap 2,048);
 *   3. optionally a coarse pass over compact keys that keeps a shortlist, followed
 *      by an exact rerank of the shortlisted original keys (LeanSparse podcast
 *      transcript, cues 07:12-08:00: 2,048 candidates, exact rerank to 512);
 *   4. sparse attention over only the selected latent rows ("Long context",
 *      paragraph "Stage 2, sparse main attention"; section "Sparsity Is a Systems
 *      Feature: The Blast Radius", "Kernel layer": a gather by token indices).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     stated otherwise.  The library allocates no memory: scratch space comes from
 *     a caller workspace whose size the matching li_*_workspace_bytes() returns.
 *   - All work is enqueued asynchronously on `stream` (NULL = the null stream);
 *     no call synchronises.  Calls on different streams do not share state.
 *     A call must not overlap another call that uses the same workspace.
 *   - Tensors are dense, row-major, contiguous; every device pointer must be
 *     16-byte aligned.
 *   - Arguments are validated on the host before anything is launched; on error
 *     nothing is launched and outputs are untouched.  No C++ exception crosses
 *     the ABI.  li_last_error() gives a human-readable reason for the last error
 *     returned on the calling thread.
 *   - Values in device arrays (nv, idx) are not validated on the host: nv entries
 *     are clamped to [0, S] by the kernels, idx entries outside [0, S) are
 *     treated as "no entry".  NaN scores are ordered above +inf (unspecified).
 *   - A top-k output is the selected set, which is unique because among equal
 *     scores the smaller key index wins, listed in ascending key index (each
 *     value beside its index).  The order carries no rank: attention over the
 *     set does not depend on it, and ascending indices keep the later gather of
 *     the selected rows sequential.  Rows with fewer than k visible keys list
 *     their visible keys, then index -1 with value -inf.
 */
#ifndef LIGHTNING_INDEXER_LI_H
#define LIGHTNING_INDEXER_LI_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum li_status {
  LI_OK = 0,
  LI_ERR_NULL = 1,      /* a required pointer is NULL                                */
  LI_ERR_SHAPE = 2,     /* a size is outside the supported range                     */
  LI_ERR_DTYPE = 3,     /* unsupported dtype or dtype combination                    */
  LI_ERR_ALIGN = 4,     /* a device pointer is not 16-byte aligned                   */
  LI_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the queried size           */
  LI_ERR_LAUNCH = 6     /* the HIP runtime reported an error when launching          */
} li_status;

typedef enum li_dtype {
  LI_F32 = 0,      /* IEEE binary32                                                  */
  LI_BF16 = 1,     /* bfloat16 (upper half of binary32), stored as 16-bit words      */
  LI_FP8_E4M3 = 2, /* OCP FP8 E4M3FN (bias 7, max 448, no inf), one byte             */
  LI_I8 = 3        /* signed 8-bit integer                                           */
} li_dtype;

/* Largest k any selection supports (the engine-side fused top-k cap of 2,048). */
#define LI_TOPK_MAX 2048
/* Indexer key width and compact key width the kernels are specialised for. */
#define LI_INDEX_DIM 128
#define LI_COMPACT_DIM 32

/* Static description of a status code (never NULL). */
const char *li_status_string(li_status s);

/* Reason for the last non-LI_OK status returned on this thread ("" if none). */
const char *li_last_error(void);

/* Library version string. */
const char *li_version(void);

/*
 * li_indexer_score -- lightning-indexer scores of every key for every query row.
 *
 *   q       [B, T, H, d]  query heads, dtype q_type in {LI_BF16, LI_F32}
 *   w       [B, T, H]     fp32 head weights (any sign)
 *   k       [B, S, d]     keys of each sequence, dtype k_type in {LI_FP8_E4M3,
 *                         LI_BF16, LI_F32}; row (b, s) is shared by all T rows of b
 *   k_scale [B, S]        fp32 per-key scale; required for LI_FP8_E4M3 (the key is
 *                         code * scale), must be NULL otherwise
 *   nv      [B*T]         int32 visible-key count per row (row r sees keys s < nv[r]);
 *                         NULL = every row sees all S keys.  This is how a causal
 *                         prefill mask is expressed.
 *   scores  [B*T, S]      fp32 output; invisible keys get -inf
 *
 * Shapes: d == 128, 1 <= H <= 128, B, T >= 1, 1 <= S < 2^31, B*T*S < 2^40.
 * Arithmetic: bf16 keys: bf16 x bf16 products, fp32 accumulation.  fp8 keys: the
 * bf16 query is split exactly into two E4M3 halves with power-of-two run scales
 * (exact for every value down to 2^-13 of its 32-value run's maximum) and each
 * half meets the key codes in the block-scaled fp8 matrix core, fp32
 * accumulation; the key scale multiplies the head sum.  All-fp32 inputs use fp32
 * FMAs.
 * Errors: LI_ERR_NULL (q, w, k, scores; k_scale for fp8), LI_ERR_SHAPE,
 * LI_ERR_DTYPE, LI_ERR_ALIGN, LI_ERR_LAUNCH.
 */
li_status li_indexer_score(const void *q, li_dtype q_type, const float *w, const void *k, li_dtype k_type,
                           const float *k_scale, const int32_t *nv, int B, int T, int S, int H, int d,
                           float *scores, hipStream_t stream);

/*
 * li_topk_select -- the k best keys of each row of a score matrix.
 *
 *   scores [R, S] fp32; nv [R] int32 or NULL (row r considers s < nv[r] only)
 *   idx    [R, k] int32 output (ascending key index, padded with -1)
 *   val    [R, k] fp32 output or NULL (the selected scores, padded with -inf)
 *   ws     workspace of at least li_topk_workspace_bytes(R, S, k) bytes (0 for
 *          shapes that need none); its contents on entry do not matter (every
 *          byte is written before it is read), and calls that share one must not
 *          overlap
 *
 * Ties are broken towards the smaller index, so the result is unique and
 * deterministic.  Shapes: R >= 1, 1 <= S < 2^31, 1 <= k <= LI_TOPK_MAX.
 * Errors: LI_ERR_NULL, LI_ERR_SHAPE, LI_ERR_ALIGN, LI_ERR_WORKSPACE, LI_ERR_LAUNCH.
 */
size_t li_topk_workspace_bytes(int R, int S, int k);
li_status li_topk_select(const float *scores, const int32_t *nv, int R, int S, int k, int32_t *idx, float *val,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * li_indexer_topk -- li_indexer_score followed by li_topk_select, with the same
 * arguments, without handing the score matrix back: for many query rows (a prefill
 * chunk) the selection runs inside the scoring kernel and the [B*T, S] scores are
 * never written to memory.  For few long rows (decode) the scoring kernel lists
 * each row's candidates above a threshold taken from a sample of its own scores,
 * and one exact pass selects among them.
 *
 *   idx [B*T, topk] int32, val [B*T, topk] fp32 or NULL (ascending key index)
 *   ws  workspace of at least li_indexer_topk_workspace_bytes(...) bytes.  The
 *       decode path keeps per-row flags there (after the score and top-k areas),
 *       which every call leaves at zero: a zero-filled workspace is ready for the
 *       first call.  Any other contents give the same results, that call being
 *       slower (its rows wait up to 200 us, then select over the whole row).
 *       Calls that share a workspace must not overlap.
 *
 * Requires q_type == LI_BF16 and k_type in {LI_BF16, LI_FP8_E4M3}, or the fp32
 * combinations accepted by li_indexer_score.  1 <= topk <= LI_TOPK_MAX.
 */
size_t li_indexer_topk_workspace_bytes(int B, int T, int S, int H, int topk);
li_status li_indexer_topk(const void *q, li_dtype q_type, const float *w, const void *k, li_dtype k_type,
                          const float *k_scale, const int32_t *nv, int B, int T, int S, int H, int d, int topk,
                          int32_t *idx, float *val, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * li_compact_search_rerank -- two-stage decode search over compact keys.
 *
 *   q        [B, H, d]   bf16 query heads (one decode row per sequence)
 *   w        [B, H]      fp32 head weights
 *   P        [dc, d]     fp32 projection shared by all sequences
 *   ck       [B, S, dc]  int8 compact keys; ck_scale [B, S] fp32 (key ~ code * scale)
 *   k_full   [B, S, d]   bf16 original keys
 *   nv       [B] int32 or NULL (= S)
 *   shortlist[B, m]      int32 output or NULL: the stage-1 shortlist, ascending key index
 *   idx      [B, k]      int32 output: the final selection, ascending key index
 *   val      [B, k]      fp64 output or NULL: the exact scores of idx
 *
 * Stage 1 projects each query head with P (fp64 fma chain over d), quantises it
 * to int8 with scale qs = max|y| / 127, sets W = w * qs (fp64), takes exact int32
 * dots D with the compact keys and scores s1 = ck_scale * sum_h W[h] max(D[h], 0)
 * (fp64 fma chain over h ascending); the m best s1 form the shortlist.  Stage 2
 * rescores the shortlisted original keys with sum_h w[h] max(q[h] . k, 0), every
 * sum an fp64 fma chain in ascending order, and keeps the k best.  Results are
 * bit-identical to a CPU evaluation of the same steps.
 * Shapes: d == 128, dc == 32, 1 <= H <= 128, 1 <= k <= m <= LI_TOPK_MAX.
 */
size_t li_compact_workspace_bytes(int B, int S, int H, int m, int k);
li_status li_compact_search_rerank(const void *q, const float *w, const float *P, const int8_t *ck,
                                   const float *ck_scale, const void *k_full, const int32_t *nv, int B, int S,
                                   int H, int d, int dc, int m, int k, int32_t *shortlist, int32_t *idx,
                                   double *val, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * li_sparse_attn_gather -- attention of every query head over only the selected
 * latent rows (MQA: one row serves all heads).
 *
 *   q    [B, Hq, dqk] bf16 queries
 *   kv   [B, S, dqk]  bf16 latent rows; keys use all dqk elements, values the first dv
 *   idx  [B, k]       int32 row indices; entries outside [0, S) (e.g. -1) are skipped
 *   out  [B, Hq, dv]  bf16 output: softmax(sm_scale * q . kv_i) weighted sum of values
 *   lse  [B, Hq]      fp32 output or NULL: log-sum-exp of the scaled logits
 *                     (-inf and a zero output when a row selects nothing)
 *   ws   workspace of at least li_sparse_attn_workspace_bytes(...) bytes
 *
 * Shapes: dqk == 576, dv == 512, 1 <= Hq <= 128 and a multiple of 32,
 * 1 <= k <= LI_TOPK_MAX.  Products are bf16 x bf16 with fp32 accumulation; the
 * softmax is evaluated in fp32 and its weights are rounded to bf16 for the
 * value product.
 */
size_t li_sparse_attn_workspace_bytes(int B, int Hq, int k, int dv);
li_status li_sparse_attn_gather(const void *q, const void *kv, const int32_t *idx, int B, int Hq, int S, int k,
                                int dqk, int dv, float sm_scale, void *out, float *lse, void *ws, size_t ws_bytes,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_INDEXER_LI_H */
