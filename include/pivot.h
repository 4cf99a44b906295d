/*
 * pivot.h -- C ABI of the PIVOT query-group indexer for MI355X (gfx950).
 *
 * PIVOT ("Proxy Indexing Via One full-prefix Traversal") replaces the dense
 * indexer of token-level sparse attention (DeepSeek Sparse Attention style).
 * Sources: the arXiv abstract of "PIVOT: Efficient Query-Group Indexing for
 * Token-Level Sparse Attention" (fugumt.com / artgrammer.co.kr paper pages)
 * and "PIVOT Explained -- From Paper to Working Code in 10 Minutes"
 * (sunghee.kr, republished by wpnews.pro), sections "How It Works" and
 * "Show Me The Code".
 *
 * Method, as computed here (one prefix scan per group):
 *   - a group is g consecutive query positions (prefill) or the g queries of
 *     one multi-token-prediction step of a sequence (decode);
 *   - its proxy query is the mean of its members: float32 sum in position
 *     order, one float32 division, rounded to the input type;
 *   - the proxy scores every key of the group's prefix [0, max(start, 1))
 *     (decode: the sequence's whole cached context) with a float32 dot
 *     product, no scale;
 *   - the candidate set C is the top K = floor(top_k * candidate_ratio) keys
 *     of that scan;
 *   - PIVOT-Refine: each member re-scores only C with its own query and
 *     keeps its own top_k; PIVOT-Reuse: every member takes the proxy's top
 *     top_k (the first top_k of C).
 *   - dense_index, for comparison: every query ranks all keys of
 *     [0, max(i, 1)) with its own scores.
 * Ranking is total: larger score first, equal scores -> smaller key index
 * first (-0.0 ranks as +0.0).
 *
 * Layouts (all row-major, contiguous, device memory):
 *   q, k        (S, H, D): element (s, h, d) at (s*H + h)*D + d
 *   q (decode)  (B*g, H, D): rows b*g .. b*g+g-1 belong to sequence b
 *   k_cache     (sum_b ctx_b, H, D): sequence b owns rows
 *               off_b .. off_b+ctx_b-1, off_b = ctx_0 + ... + ctx_{b-1}
 *   out_idx     (rows, H, top_k) int32: row (i, h) lists the selected key
 *               indices (relative to the sequence) best first; slots past
 *               the valid count hold -1
 *   out_score   optional, same shape, float32: the score that ranked each
 *               slot (Reuse: proxy score; Refine and dense: the query's own
 *               score); padding holds -inf
 *   Valid counts: Refine min(top_k, min(K, n)), Reuse min(top_k, n),
 *   dense min(top_k, max(i, 1)), with n the group's prefix length.
 *   Alignment: q, k, k_cache, v and the workspace start on 16-byte
 *   boundaries, int32 / float32 arrays on 4-byte boundaries (PIVOT_EINVAL,
 *   or PIVOT_EWORKSPACE for the workspace, otherwise).
 *
 * Ownership and execution: the caller owns every buffer; the library never
 * allocates device memory and keeps no state between calls (apart from the
 * optional stage-timing records below). Work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 * call returns once it is enqueued. Calls are reentrant for distinct
 * workspaces, except while stage timing is enabled (pivot_profile_enable):
 * the timing records are process-wide, so calls from several threads must
 * then be serialised. The workspace is scratch device memory of at least the size
 * the matching *_workspace_bytes function returns; a smaller workspace that
 * still holds one head's share is used in several passes over the heads.
 *
 * Errors: every argument check runs on the host before anything is
 * enqueued; on error nothing is written. Status codes, never exceptions.
 */
#ifndef PIVOT_H
#define PIVOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PIVOT_OK = 0,
    PIVOT_EINVAL = -1,      /* bad pointer, size or parameter */
    PIVOT_EUNSUPPORTED = -2,/* valid but outside what the kernels handle */
    PIVOT_EWORKSPACE = -3,  /* workspace too small (or NULL) */
    PIVOT_EHIP = -4         /* a HIP launch or runtime call failed */
} pivot_status;

typedef enum { PIVOT_F32 = 0, PIVOT_BF16 = 1 } pivot_dtype;
/* PIVOT_REFINE_LITERAL (prefill only, for comparison): the per-position
 * rescan that the pivot_refine code of "PIVOT Explained", section "Show Me
 * The Code", carries out as written -- position i >= 1 scans keys [0, i)
 * with its group's proxy, takes its own min(K, i) candidates and re-scores
 * them with q_i; position 0 (skipped by that code) is all padding. It does g
 * scans per group where PIVOT_REFINE does one. */
typedef enum { PIVOT_REFINE = 0, PIVOT_REUSE = 1, PIVOT_REFINE_LITERAL = 2 } pivot_mode;

/* Downstream sparse attention over indexer rows -- the attention the pages
 * run on the indices ("PIVOT Explained", "Show Me The Code", quick test):
 *   out[i, h, :] = sum_c w_c v[c, h, :],
 *   w_c = exp(scale q[i,h,:].k[c,h,:]) / sum_c' exp(scale q[i,h,:].k[c',h,:])
 * over the entries c of idx[i, h, :] that lie in [0, S) (-1 and anything
 * else is padding; repeated entries count each time); a row with no such
 * entry is zero. Scores, softmax and the weighted sum run in float32.
 *   q, k, v  device (S, H, D) of `dtype`, D in {64, 128}
 *   idx      device (S, H, top_k) int32 (an indexer's output, or any rows)
 *   scale    finite; the pages use D^-0.5
 *   out      device (S, H, D) float32, written completely
 * Errors as above; no workspace. */
int pivot_sparse_attention(const void *q, const void *k, const void *v,
                           int32_t dtype, int64_t S, int32_t H, int32_t D,
                           const int32_t *idx, int32_t top_k, float scale,
                           float *out, void *stream);

/* The same attention for rows shared by groups of g consecutive positions
 * (the rows PIVOT-Reuse returns: every member of a group has the row of its
 * first position): positions j*g .. min(j*g + g, S) - 1 all attend over the
 * index row of position j*g, which is read once per group; the other rows of
 * idx are not read. Each group's key and value rows are gathered once for
 * all of its members. Arguments and errors as for pivot_sparse_attention,
 * plus g >= 1; the output is the attention above for every position. */
int pivot_sparse_attention_grouped(const void *q, const void *k, const void *v,
                                   int32_t dtype, int64_t S, int32_t H,
                                   int32_t D, const int32_t *idx,
                                   int32_t top_k, int32_t g, float scale,
                                   float *out, void *stream);

/* Human-readable text of a status code (static storage). */
const char *pivot_status_string(int status);

/* K = floor(top_k * candidate_ratio) as the pages' int(top_k * ratio)
 * ("Show Me The Code"). Writes K and returns PIVOT_OK, or PIVOT_EINVAL when
 * top_k < 1, ratio is not positive/finite or K < top_k. */
int pivot_candidate_count(int32_t top_k, double candidate_ratio, int64_t *K_out);

/* Workspace for pivot_index_prefill processing all H heads in one pass.
 * Returns 0 for invalid arguments. Query with H = 1 for the smallest
 * workspace accepted (one head per pass). */
size_t pivot_prefill_workspace_bytes(int64_t S, int32_t H, int32_t D,
                                     int32_t top_k, int32_t g,
                                     double candidate_ratio, int32_t mode,
                                     int32_t dtype);

/* Prefill indexer (abstract: fixed-size groups of consecutive queries).
 *   q, k      device (S, H, D) of `dtype` (PIVOT_F32 or PIVOT_BF16)
 *   S >= 1, H >= 1, D in {64, 128}, 1 <= top_k <= 8192, g >= 1,
 *   K = floor(top_k * candidate_ratio) with top_k <= K <= 8192 (the
 *   resource limit of the selection kernels; larger -> PIVOT_EUNSUPPORTED),
 *   mode      PIVOT_REFINE, PIVOT_REUSE or PIVOT_REFINE_LITERAL
 *   The scan reads 32 sampled key rows at 32-bit offsets from the first:
 *   inputs where 32 * s * H * D * element size reaches 4 GiB (s, the
 *   sampling stride, is about S / 4080 for long sequences) return
 *   PIVOT_EUNSUPPORTED; no input that fits one GPU's memory comes near. 
 *   out_idx   device (S, H, top_k) int32, written completely
 *   out_score device (S, H, top_k) float32 or NULL
 *   workspace device scratch, workspace_bytes as described above
 *   stream    hipStream_t or NULL */
int pivot_index_prefill(const void *q, const void *k, int32_t dtype, int64_t S,
                        int32_t H, int32_t D, int32_t top_k, int32_t g,
                        double candidate_ratio, int32_t mode, int32_t *out_idx,
                        float *out_score, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Workspace for pivot_index_decode; ctx_lens_host is host memory (B
 * entries, each >= 1). Returns 0 for invalid arguments. */
size_t pivot_decode_workspace_bytes(int32_t B, const int64_t *ctx_lens_host,
                                    int32_t g, int32_t H, int32_t D,
                                    int32_t top_k, double candidate_ratio,
                                    int32_t mode, int32_t dtype);

/* Decode indexer (abstract: the queries decoded together in one MTP step
 * form a group). Sequence b's g queries are rows b*g .. b*g+g-1 of q and
 * scan its whole cached context [0, ctx_b).
 *   q             device (B*g, H, D) of dtype
 *   k_cache       device (sum ctx, H, D) of dtype, packed by sequence
 *   ctx_lens_host host int64[B], each 1 <= ctx_b < 2^31; read during the
 *                 call only
 *   B >= 1, g >= 1; other limits as for prefill
 *   out_idx       device (B*g, H, top_k) int32; out_score as for prefill */
int pivot_index_decode(const void *q, const void *k_cache, int32_t dtype,
                       const int64_t *ctx_lens_host, int32_t B, int32_t g,
                       int32_t H, int32_t D, int32_t top_k,
                       double candidate_ratio, int32_t mode, int32_t *out_idx,
                       float *out_score, void *workspace,
                       size_t workspace_bytes, void *stream);

/* pivot_index_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, results and errors as
 * pivot_index_decode, without the workspace. The scratch is the library's
 * own static device array of 256 MiB (one copy per GPU, held until the
 * process ends; the 64-sequence decode step with contexts up to 131072, H =
 * 8, D = 128, top_k = 2048, K = 4096 needs 222 MiB of it). A call whose
 * pivot_decode_workspace_bytes exceeds 256 MiB returns PIVOT_EWORKSPACE
 * before anything is enqueued. The call allocates nothing and records no
 * stage-timing events. Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller. The first call on a device looks the
 * array's address up (hipGetSymbolAddress) with that device current. */
int pivot_index_decode_noalloc(const void *q, const void *k_cache,
                               int32_t dtype, const int64_t *ctx_lens_host,
                               int32_t B, int32_t g, int32_t H, int32_t D,
                               int32_t top_k, double candidate_ratio,
                               int32_t mode, int32_t *out_idx,
                               float *out_score, void *stream);

/* Workspace for dense_index (all heads in one pass; H = 1 gives the
 * minimum). Returns 0 for invalid arguments. */
size_t dense_index_workspace_bytes(int64_t S, int32_t H, int32_t D,
                                   int32_t top_k, int32_t dtype);

/* Dense indexer, for comparison (abstract: score every preceding token and
 * keep the top-k; "The Problem" section of "PIVOT Explained"): row (i, h)
 * ranks keys [0, max(i, 1)) by q[i, h] . k[c, h]. Arguments as for prefill;
 * 1 <= top_k <= 8192. */
int dense_index(const void *q, const void *k, int32_t dtype, int64_t S,
                int32_t H, int32_t D, int32_t top_k, int32_t *out_idx,
                float *out_score, void *workspace, size_t workspace_bytes,
                void *stream);

/* Stage timing, for benchmarking and tracing. While enabled, every call
 * records a pair of HIP events on its stream around each kernel stage.
 * pivot_profile_read waits for the recorded events, adds each stage's
 * elapsed milliseconds and launch count into ms_out[stage] / count_out[stage]
 * (arrays of n_stages entries, first zeroed by the call) and forgets the
 * records. Stages: 0 proxy mean, 1 sample scan, 2 thresholds, 3 main scan,
 * 4 select, 5 exact fallback, 6 refine, 7 decode scan, 8 decode select.
 * At most 8192 records are kept between reads (later ones are dropped).
 * Not thread-safe: one benchmarking thread only. Returns PIVOT_OK, or
 * PIVOT_EINVAL / PIVOT_EHIP. */
#define PIVOT_N_STAGES 9
int pivot_profile_enable(int on);
int pivot_profile_read(double *ms_out, int64_t *count_out, int n_stages);

#ifdef __cplusplus
}
#endif

#endif /* PIVOT_H */
