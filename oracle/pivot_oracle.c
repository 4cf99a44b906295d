/*
 * PIVOT query-group indexer -- plain CPU oracle.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load this library. The product path (the HIP library
 * and its Python binding) never calls it, and this file shares no code,
 * header, table or helper with the GPU path.
 *
 * Sources: "PIVOT Explained -- From Paper to Working Code in 10 Minutes"
 * (sunghee.kr, republished on wpnews.pro), sections "How It Works" (the
 * algorithm listing) and "Show Me The Code" (pivot_refine / pivot_reuse), and
 * the arXiv abstract of "PIVOT: Efficient Query-Group Indexing for Token-Level
 * Sparse Attention" (fugumt.com and artgrammer.co.kr paper pages).
 *
 * Everything here is written for a reader to check by eye against those
 * pages: one proxy per group, one causal prefix scan per group, a full sort of
 * the prefix under a total order, then Reuse (share the proxy's top-k) or
 * Refine (re-score the candidate set per query). No blocking, no fusion, no
 * early exits. Scores accumulate in double and are rounded once to float.
 *
 * Readings of points the pages leave open (each one also listed in the
 * design notes of the repository):
 *   - one prefix scan per group over keys [0, max(group_start, 1)), for both
 *     variants (the listing in "How It Works" and the abstract; the Reuse code
 *     uses exactly this prefix, the Refine code's per-position rescan is the
 *     illustrative variant and is not what is computed here);
 *   - total order: larger score first, equal scores -> smaller key index
 *     first; -0.0 is treated as +0.0;
 *   - K = floor(top_k * candidate_ratio) computed in double, as the code's
 *     int(top_k * candidate_ratio); K < top_k is rejected;
 *   - the proxy is a float32 sequential sum in ascending position, one IEEE
 *     float32 division by the group size, then round-to-nearest-even to the
 *     input type (bf16 inputs give a bf16 proxy, as torch's mean does);
 *   - scores carry no 1/sqrt(D) scale (that scale only appears in the
 *     downstream attention demo of "Show Me The Code");
 *   - padding slots hold index -1 and score -inf (the pages zero-fill,
 *     which collides with key 0);
 *   - dense indexer: query i ranks keys [0, max(i, 1)) by its own score;
 *   - decode: the g queries of one multi-token-prediction step of sequence b
 *     form one group whose prefix is the whole cached context [0, ctx_b),
 *     ctx_b >= 1;
 *   - the literal per-position Refine (mode 2, kept for comparison): the
 *     pivot_refine code of "Show Me The Code" as written -- position i >= 1
 *     scans keys [0, i) with its group's proxy, takes its own candidate set
 *     and re-scores it with q_i; position 0, which that code skips, gets a
 *     row of padding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_REFINE 0
#define OR_REUSE 1
#define OR_REFINE_LITERAL 2

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENOMEM (-2)

/* ---------------------------------------------------------------- numbers */

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest-even from float32 to bf16 (finite inputs only). */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* Element at flat offset `off` of an (S, H, D) tensor stored as dtype `dt`. */
static float load_elem(const void *base, int dt, size_t off)
{
    if (dt == OR_BF16)
        return bf16_to_float(((const uint16_t *)base)[off]);
    return ((const float *)base)[off];
}

/* Indexer score of key row `krow` (D contiguous elements at flat offset
 * `koff`) against vector `a`: the exact-as-possible dot product (double
 * accumulation, each product exact for bf16/fp32 operands), rounded once to
 * float32. No scale. -0.0 is returned as +0.0. */
static float score_of(const float *a, const void *k, int dt, size_t koff, int D)
{
    double acc = 0.0;
    for (int d = 0; d < D; ++d)
        acc += (double)a[d] * (double)load_elem(k, dt, koff + (size_t)d);
    float s = (float)acc;
    if (s == 0.0f)
        s = 0.0f;
    return s;
}

/* ------------------------------------------------------------ total order */

typedef struct {
    float score;
    int32_t idx;
} scored_t;

/* qsort comparator: better entries first (score descending, index
 * ascending). Scores are finite and never -0.0 here. */
static int better_first(const void *pa, const void *pb)
{
    const scored_t *a = (const scored_t *)pa;
    const scored_t *b = (const scored_t *)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    if (a->idx < b->idx)
        return -1;
    if (a->idx > b->idx)
        return 1;
    return 0;
}

static void write_row(int32_t *out_idx, float *out_score, size_t row_off,
                      int top_k, const scored_t *best, int64_t n_valid)
{
    for (int t = 0; t < top_k; ++t) {
        if (t < n_valid) {
            out_idx[row_off + t] = best[t].idx;
            if (out_score)
                out_score[row_off + t] = best[t].score;
        } else {
            out_idx[row_off + t] = -1;
            if (out_score)
                out_score[row_off + t] = -INFINITY;
        }
    }
}

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

/* ------------------------------------------------------------- parameters */

/* K = int(top_k * candidate_ratio), the candidate-set size of the code in
 * "Show Me The Code". Returns -1 when K would fall below top_k or the inputs
 * are not positive. */
int64_t oracle_candidate_count(int32_t top_k, double candidate_ratio)
{
    if (top_k < 1 || !(candidate_ratio > 0.0))
        return -1;
    double prod = (double)top_k * candidate_ratio;
    if (prod > 9.0e18)
        return -1;
    int64_t K = (int64_t)floor(prod);
    if (K < top_k)
        return -1;
    return K;
}

/* ------------------------------------------------------------------ proxy */

/* Proxy query of one group (the mean of its member queries, "How It Works"):
 * members are rows i0 .. i0+m-1 of q (row stride H*D), head h. */
static void group_proxy(const void *q, int dt, int H, int D, int h, int64_t i0,
                        int64_t m, float *p)
{
    for (int d = 0; d < D; ++d) {
        float sum = 0.0f;
        for (int64_t i = i0; i < i0 + m; ++i)
            sum += load_elem(q, dt, ((size_t)i * H + h) * D + d);
        float v = sum / (float)m;
        if (dt == OR_BF16)
            v = bf16_to_float(float_to_bf16_rne(v));
        p[d] = v;
    }
}

/* Exposed for tests: the proxy of group j of head h of a prefill. */
int oracle_proxy(const void *q, int dt, int64_t S, int32_t H, int32_t D,
                 int32_t g, int32_t h, int64_t j, float *out_p)
{
    if (!q || !out_p || S < 1 || H < 1 || D < 1 || g < 1 || h < 0 || h >= H)
        return OR_EINVAL;
    int64_t i0 = j * (int64_t)g;
    if (j < 0 || i0 >= S)
        return OR_EINVAL;
    group_proxy(q, dt, H, D, h, i0, min64(g, S - i0), out_p);
    return OR_OK;
}

/* --------------------------------------------------------------- one group */

/* The shared work of one group (prefill group or decode step):
 *   members: query rows qi0 .. qi0+m-1 of q (row stride H*D), head h;
 *   prefix:  key rows kbase .. kbase+n-1 of k (row stride H*D), head h;
 *   outputs: rows out_row0 .. out_row0+m-1 of (rows, H, top_k).
 * Follows "How It Works": proxy = mean(group); scores = proxy . K[prefix];
 * C = top-K(scores); Reuse keeps C's first top_k for every member, Refine
 * re-scores C with each member and keeps that member's own top_k.
 * When cand_out is given, C (in order) is copied there as well. */
static int one_group(const void *q, const void *k, int dt, int H, int D,
                     int top_k, int64_t K, int mode, int h, int64_t qi0,
                     int64_t m, int64_t kbase, int64_t n, int32_t *out_idx,
                     float *out_score, int64_t out_row0, scored_t *cand_out,
                     int64_t *n_cand_out)
{
    float *p = (float *)malloc(sizeof(float) * (size_t)D);
    float *a = (float *)malloc(sizeof(float) * (size_t)D);
    scored_t *all = (scored_t *)malloc(sizeof(scored_t) * (size_t)n);
    int64_t nc = min64(K, n);
    scored_t *mine = (scored_t *)malloc(sizeof(scored_t) * (size_t)nc);
    if (!p || !a || !all || !mine) {
        free(p);
        free(a);
        free(all);
        free(mine);
        return OR_ENOMEM;
    }

    /* proxy query and the one causal prefix scan of the group */
    group_proxy(q, dt, H, D, h, qi0, m, p);
    for (int64_t c = 0; c < n; ++c) {
        all[c].score = score_of(p, k, dt, ((size_t)(kbase + c) * H + h) * D, D);
        all[c].idx = (int32_t)c;
    }
    /* candidate set C = the first min(K, n) keys under the total order */
    qsort(all, (size_t)n, sizeof(scored_t), better_first);
    if (cand_out)
        memcpy(cand_out, all, sizeof(scored_t) * (size_t)nc);
    if (n_cand_out)
        *n_cand_out = nc;

    int64_t n_valid = min64(top_k, nc);
    for (int64_t t = 0; t < m; ++t) {
        size_t row_off = ((size_t)(out_row0 + t) * H + h) * (size_t)top_k;
        if (!out_idx)
            break;
        if (mode == OR_REUSE) {
            /* PIVOT-Reuse: every member shares the proxy's top entries */
            write_row(out_idx, out_score, row_off, top_k, all, n_valid);
        } else {
            /* PIVOT-Refine: re-score only the candidates with this query */
            for (int d = 0; d < D; ++d)
                a[d] = load_elem(q, dt, ((size_t)(qi0 + t) * H + h) * D + d);
            for (int64_t c = 0; c < nc; ++c) {
                int32_t key = all[c].idx;
                mine[c].score =
                    score_of(a, k, dt, ((size_t)(kbase + key) * H + h) * D, D);
                mine[c].idx = key;
            }
            qsort(mine, (size_t)nc, sizeof(scored_t), better_first);
            write_row(out_idx, out_score, row_off, top_k, mine, n_valid);
        }
    }
    free(p);
    free(a);
    free(all);
    free(mine);
    return OR_OK;
}

/* The literal per-position Refine row of position i, head h (the pivot_refine
 * code of "Show Me The Code"): the proxy of i's group scans keys [0, i), the
 * first min(K, i) under the total order are i's candidates, q_i re-scores
 * them and keeps its own first min(top_k, |C|). Position 0 is skipped by that
 * code: its row is all padding. */
static int literal_row(const void *q, const void *k, int dt, int64_t S, int H, int D,
                       int top_k, int64_t K, int g, int h, int64_t i,
                       int32_t *out_idx, float *out_score, size_t row_off)
{
    if (i == 0) {
        write_row(out_idx, out_score, row_off, top_k, NULL, 0);
        return OR_OK;
    }
    int64_t i0 = (i / g) * (int64_t)g;
    int64_t m = min64(g, S - i0);
    int64_t n = i;
    int64_t nc = min64(K, n);
    float *p = (float *)malloc(sizeof(float) * (size_t)D);
    float *a = (float *)malloc(sizeof(float) * (size_t)D);
    scored_t *all = (scored_t *)malloc(sizeof(scored_t) * (size_t)n);
    scored_t *mine = (scored_t *)malloc(sizeof(scored_t) * (size_t)nc);
    if (!p || !a || !all || !mine) {
        free(p);
        free(a);
        free(all);
        free(mine);
        return OR_ENOMEM;
    }
    group_proxy(q, dt, H, D, h, i0, m, p);
    for (int64_t c = 0; c < n; ++c) {
        all[c].score = score_of(p, k, dt, ((size_t)c * H + h) * D, D);
        all[c].idx = (int32_t)c;
    }
    qsort(all, (size_t)n, sizeof(scored_t), better_first);
    for (int d = 0; d < D; ++d)
        a[d] = load_elem(q, dt, ((size_t)i * H + h) * D + d);
    for (int64_t c = 0; c < nc; ++c) {
        int32_t key = all[c].idx;
        mine[c].score = score_of(a, k, dt, ((size_t)key * H + h) * D, D);
        mine[c].idx = key;
    }
    qsort(mine, (size_t)nc, sizeof(scored_t), better_first);
    write_row(out_idx, out_score, row_off, top_k, mine, min64(top_k, nc));
    free(p);
    free(a);
    free(all);
    free(mine);
    return OR_OK;
}

/* The dense indexer row of query i, head h: rank every key of [0, max(i,1))
 * by q_i's own score (the DSA indexer the pages compare against). */
static int dense_row(const void *q, const void *k, int dt, int H, int D,
                     int top_k, int h, int64_t i, int32_t *out_idx,
                     float *out_score, size_t row_off)
{
    int64_t n = max64(i, 1);
    float *a = (float *)malloc(sizeof(float) * (size_t)D);
    scored_t *all = (scored_t *)malloc(sizeof(scored_t) * (size_t)n);
    if (!a || !all) {
        free(a);
        free(all);
        return OR_ENOMEM;
    }
    for (int d = 0; d < D; ++d)
        a[d] = load_elem(q, dt, ((size_t)i * H + h) * D + d);
    for (int64_t c = 0; c < n; ++c) {
        all[c].score = score_of(a, k, dt, ((size_t)c * H + h) * D, D);
        all[c].idx = (int32_t)c;
    }
    qsort(all, (size_t)n, sizeof(scored_t), better_first);
    write_row(out_idx, out_score, row_off, top_k, all, min64(top_k, n));
    free(a);
    free(all);
    return OR_OK;
}

static int check_common(const void *q, const void *k, int dt, int64_t S,
                        int32_t H, int32_t D, int32_t top_k)
{
    if (!q || !k || S < 1 || H < 1 || D < 1 || top_k < 1)
        return OR_EINVAL;
    if (dt != OR_F32 && dt != OR_BF16)
        return OR_EINVAL;
    if (S > INT32_MAX)
        return OR_EINVAL;
    return OR_OK;
}

/* ------------------------------------------------------------ public API */

/* Prefill indexer for heads [h_begin, h_end): writes those heads' slots of
 * out_idx / out_score, both shaped (S, H, top_k); other heads untouched.
 * Groups are consecutive positions [j*g, min(j*g+g, S)); group j scans keys
 * [0, max(j*g, 1)). */
int oracle_prefill(const void *q, const void *k, int dt, int64_t S, int32_t H,
                   int32_t D, int32_t top_k, int32_t g, double candidate_ratio,
                   int mode, int32_t h_begin, int32_t h_end, int32_t *out_idx,
                   float *out_score)
{
    int rc = check_common(q, k, dt, S, H, D, top_k);
    if (rc)
        return rc;
    int64_t K = oracle_candidate_count(top_k, candidate_ratio);
    if (K < 0 || g < 1 || !out_idx ||
        (mode != OR_REFINE && mode != OR_REUSE && mode != OR_REFINE_LITERAL))
        return OR_EINVAL;
    if (h_begin < 0 || h_end > H || h_begin > h_end)
        return OR_EINVAL;
    if (mode == OR_REFINE_LITERAL) {
        for (int32_t h = h_begin; h < h_end; ++h)
            for (int64_t i = 0; i < S; ++i) {
                rc = literal_row(q, k, dt, S, H, D, top_k, K, g, h, i, out_idx, out_score,
                                 ((size_t)i * H + h) * (size_t)top_k);
                if (rc)
                    return rc;
            }
        return OR_OK;
    }
    for (int32_t h = h_begin; h < h_end; ++h) {
        for (int64_t i0 = 0; i0 < S; i0 += g) {
            int64_t m = min64(g, S - i0);
            int64_t n = max64(i0, 1);
            rc = one_group(q, k, dt, H, D, top_k, K, mode, h, i0, m, 0, n,
                           out_idx, out_score, i0, NULL, NULL);
            if (rc)
                return rc;
        }
    }
    return OR_OK;
}

/* Prefill indexer for selected (position, head) rows only: row r of the
 * outputs (shaped (n_rows, top_k)) is the indexer row of position rows_i[r],
 * head rows_h[r]. The group of each row is recomputed in full. */
int oracle_prefill_rows(const void *q, const void *k, int dt, int64_t S,
                        int32_t H, int32_t D, int32_t top_k, int32_t g,
                        double candidate_ratio, int mode, int64_t n_rows,
                        const int64_t *rows_i, const int32_t *rows_h,
                        int32_t *out_idx, float *out_score)
{
    int rc = check_common(q, k, dt, S, H, D, top_k);
    if (rc)
        return rc;
    int64_t K = oracle_candidate_count(top_k, candidate_ratio);
    if (K < 0 || g < 1 || !out_idx || !rows_i || !rows_h || n_rows < 0 ||
        (mode != OR_REFINE && mode != OR_REUSE && mode != OR_REFINE_LITERAL))
        return OR_EINVAL;
    if (mode == OR_REFINE_LITERAL) {
        for (int64_t r = 0; r < n_rows; ++r) {
            if (rows_i[r] < 0 || rows_i[r] >= S || rows_h[r] < 0 || rows_h[r] >= H)
                return OR_EINVAL;
            rc = literal_row(q, k, dt, S, H, D, top_k, K, g, rows_h[r], rows_i[r], out_idx, out_score,
                             (size_t)r * top_k);
            if (rc)
                return rc;
        }
        return OR_OK;
    }
    int32_t *tmp_idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)g * H * top_k);
    float *tmp_sc = (float *)malloc(sizeof(float) * (size_t)g * H * top_k);
    if (!tmp_idx || !tmp_sc) {
        free(tmp_idx);
        free(tmp_sc);
        return OR_ENOMEM;
    }
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = rows_i[r];
        int32_t h = rows_h[r];
        if (i < 0 || i >= S || h < 0 || h >= H) {
            rc = OR_EINVAL;
            break;
        }
        int64_t i0 = (i / g) * g;
        int64_t m = min64(g, S - i0);
        /* outputs of this group land in a (g, H, top_k) scratch at row 0 */
        rc = one_group(q, k, dt, H, D, top_k, K, mode, h, i0, m, 0,
                       max64(i0, 1), tmp_idx, tmp_sc, 0, NULL, NULL);
        if (rc)
            break;
        size_t src = ((size_t)(i - i0) * H + h) * (size_t)top_k;
        memcpy(out_idx + (size_t)r * top_k, tmp_idx + src, sizeof(int32_t) * (size_t)top_k);
        if (out_score)
            memcpy(out_score + (size_t)r * top_k, tmp_sc + src, sizeof(float) * (size_t)top_k);
    }
    free(tmp_idx);
    free(tmp_sc);
    return rc;
}

/* Whole groups of a prefill: group (heads[t], groups[t]) for t < n_groups,
 * every member row written to out_idx / out_score shaped (n_groups, g,
 * top_k) (rows past a ragged last group stay -1 / -inf). */
int oracle_prefill_groups(const void *q, const void *k, int dt, int64_t S,
                          int32_t H, int32_t D, int32_t top_k, int32_t g,
                          double candidate_ratio, int mode, int64_t n_groups,
                          const int32_t *heads, const int64_t *groups,
                          int32_t *out_idx, float *out_score)
{
    int rc = check_common(q, k, dt, S, H, D, top_k);
    if (rc)
        return rc;
    int64_t K = oracle_candidate_count(top_k, candidate_ratio);
    if (K < 0 || g < 1 || !out_idx || !heads || !groups || n_groups < 0 ||
        (mode != OR_REFINE && mode != OR_REUSE))
        return OR_EINVAL;
    size_t one = (size_t)g * H * top_k;
    int32_t *tmp_idx = (int32_t *)malloc(sizeof(int32_t) * one);
    float *tmp_sc = (float *)malloc(sizeof(float) * one);
    if (!tmp_idx || !tmp_sc) {
        free(tmp_idx);
        free(tmp_sc);
        return OR_ENOMEM;
    }
    for (int64_t t = 0; t < n_groups && rc == OR_OK; ++t) {
        int32_t h = heads[t];
        int64_t i0 = groups[t] * (int64_t)g;
        if (h < 0 || h >= H || groups[t] < 0 || i0 >= S) {
            rc = OR_EINVAL;
            break;
        }
        int64_t m = min64(g, S - i0);
        rc = one_group(q, k, dt, H, D, top_k, K, mode, h, i0, m, 0, max64(i0, 1),
                       tmp_idx, tmp_sc, 0, NULL, NULL);
        for (int64_t u = 0; u < g && rc == OR_OK; ++u) {
            size_t dst = ((size_t)t * g + u) * (size_t)top_k;
            size_t src = ((size_t)u * H + h) * (size_t)top_k;
            for (int c = 0; c < top_k; ++c) {
                out_idx[dst + c] = u < m ? tmp_idx[src + c] : -1;
                if (out_score)
                    out_score[dst + c] = u < m ? tmp_sc[src + c] : -INFINITY;
            }
        }
    }
    free(tmp_idx);
    free(tmp_sc);
    return rc;
}

/* Candidate set C of group j, head h of a prefill, in total order: writes
 * min(K, n_j) indices (and their proxy scores) and returns that count, or a
 * negative error. */
int64_t oracle_prefill_candidates(const void *q, const void *k, int dt,
                                  int64_t S, int32_t H, int32_t D,
                                  int32_t top_k, int32_t g,
                                  double candidate_ratio, int32_t h, int64_t j,
                                  int32_t *out_cand, float *out_score)
{
    int rc = check_common(q, k, dt, S, H, D, top_k);
    if (rc)
        return rc;
    int64_t K = oracle_candidate_count(top_k, candidate_ratio);
    if (K < 0 || g < 1 || !out_cand || h < 0 || h >= H || j < 0)
        return OR_EINVAL;
    int64_t i0 = j * (int64_t)g;
    if (i0 >= S)
        return OR_EINVAL;
    int64_t n = max64(i0, 1);
    scored_t *cand = (scored_t *)malloc(sizeof(scored_t) * (size_t)min64(K, n));
    if (!cand)
        return OR_ENOMEM;
    int64_t nc = 0;
    rc = one_group(q, k, dt, H, D, top_k, K, OR_REUSE, h, i0, min64(g, S - i0),
                   0, n, NULL, NULL, 0, cand, &nc);
    if (rc == OR_OK) {
        for (int64_t t = 0; t < nc; ++t) {
            out_cand[t] = cand[t].idx;
            if (out_score)
                out_score[t] = cand[t].score;
        }
    }
    free(cand);
    return rc ? rc : nc;
}

/* Dense indexer for heads [h_begin, h_end); outputs shaped (S, H, top_k). */
int oracle_dense(const void *q, const void *k, int dt, int64_t S, int32_t H,
                 int32_t D, int32_t top_k, int32_t h_begin, int32_t h_end,
                 int32_t *out_idx, float *out_score)
{
    int rc = check_common(q, k, dt, S, H, D, top_k);
    if (rc)
        return rc;
    if (!out_idx || h_begin < 0 || h_end > H || h_begin > h_end)
        return OR_EINVAL;
    for (int32_t h = h_begin; h < h_end; ++h)
        for (int64_t i = 0; i < S; ++i) {
            rc = dense_row(q, k, dt, H, D, top_k, h, i, out_idx, out_score,
                           ((size_t)i * H + h) * (size_t)top_k);
            if (rc)
                return rc;
        }
    return OR_OK;
}

/* Dense indexer for selected rows; outputs shaped (n_rows, top_k). */
int oracle_dense_rows(const void *q, const void *k, int dt, int64_t S,
                      int32_t H, int32_t D, int32_t top_k, int64_t n_rows,
                      const int64_t *rows_i, const int32_t *rows_h,
                      int32_t *out_idx, float *out_score)
{
    int rc = check_common(q, k, dt, S, H, D, top_k);
    if (rc)
        return rc;
    if (!out_idx || !rows_i || !rows_h || n_rows < 0)
        return OR_EINVAL;
    for (int64_t r = 0; r < n_rows; ++r) {
        if (rows_i[r] < 0 || rows_i[r] >= S || rows_h[r] < 0 || rows_h[r] >= H)
            return OR_EINVAL;
        rc = dense_row(q, k, dt, H, D, top_k, rows_h[r], rows_i[r], out_idx,
                       out_score, (size_t)r * top_k);
        if (rc)
            return rc;
    }
    return OR_OK;
}

/* Decode indexer for heads [h_begin, h_end). Sequence b owns the g query rows
 * b*g .. b*g+g-1 of q, shaped (B*g, H, D), and the cache rows
 * off_b .. off_b+ctx_b-1 of k_cache, shaped (sum ctx, H, D), where off_b is
 * the sum of the earlier context lengths. Its g queries form one group whose
 * prefix is its whole cached context (abstract: decode groups are the
 * queries of one multi-token-prediction step). Outputs (B*g, H, top_k). */
int oracle_decode(const void *q, const void *k_cache, int dt,
                  const int64_t *ctx_lens, int32_t B, int32_t g, int32_t H,
                  int32_t D, int32_t top_k, double candidate_ratio, int mode,
                  int32_t h_begin, int32_t h_end, int32_t *out_idx,
                  float *out_score)
{
    if (!q || !k_cache || !ctx_lens || !out_idx || B < 1 || g < 1 || H < 1 ||
        D < 1 || top_k < 1 || (dt != OR_F32 && dt != OR_BF16) ||
        (mode != OR_REFINE && mode != OR_REUSE))
        return OR_EINVAL;
    if (h_begin < 0 || h_end > H || h_begin > h_end)
        return OR_EINVAL;
    int64_t K = oracle_candidate_count(top_k, candidate_ratio);
    if (K < 0)
        return OR_EINVAL;
    for (int32_t b = 0; b < B; ++b)
        if (ctx_lens[b] < 1 || ctx_lens[b] > INT32_MAX)
            return OR_EINVAL;
    for (int32_t h = h_begin; h < h_end; ++h) {
        int64_t off = 0;
        for (int32_t b = 0; b < B; ++b) {
            int rc = one_group(q, k_cache, dt, H, D, top_k, K, mode, h,
                               (int64_t)b * g, g, off, ctx_lens[b], out_idx,
                               out_score, (int64_t)b * g, NULL, NULL);
            if (rc)
                return rc;
            off += ctx_lens[b];
        }
    }
    return OR_OK;
}

/* Candidate set C of sequence b, head h of a decode step (layouts as for
 * oracle_decode), in total order: writes min(K, ctx_b) indices relative to
 * the sequence (and their proxy scores) and returns that count, or a
 * negative error. */
int64_t oracle_decode_candidates(const void *q, const void *k_cache, int dt,
                                 const int64_t *ctx_lens, int32_t B, int32_t g,
                                 int32_t H, int32_t D, int32_t top_k,
                                 double candidate_ratio, int32_t h, int32_t b,
                                 int32_t *out_cand, float *out_score)
{
    if (!q || !k_cache || !ctx_lens || !out_cand || B < 1 || g < 1 || H < 1 ||
        D < 1 || top_k < 1 || (dt != OR_F32 && dt != OR_BF16) || h < 0 ||
        h >= H || b < 0 || b >= B)
        return OR_EINVAL;
    int64_t K = oracle_candidate_count(top_k, candidate_ratio);
    if (K < 0)
        return OR_EINVAL;
    int64_t off = 0;
    for (int32_t t = 0; t < b; ++t)
        off += ctx_lens[t];
    int64_t n = ctx_lens[b];
    if (n < 1)
        return OR_EINVAL;
    scored_t *cand = (scored_t *)malloc(sizeof(scored_t) * (size_t)min64(K, n));
    if (!cand)
        return OR_ENOMEM;
    int64_t nc = 0;
    int rc = one_group(q, k_cache, dt, H, D, top_k, K, OR_REUSE, h, (int64_t)b * g,
                       g, off, n, NULL, NULL, 0, cand, &nc);
    if (rc == OR_OK) {
        for (int64_t t = 0; t < nc; ++t) {
            out_cand[t] = cand[t].idx;
            if (out_score)
                out_score[t] = cand[t].score;
        }
    }
    free(cand);
    return rc ? rc : nc;
}

/* ---------------------------------------------- downstream sparse attention */

/* The attention the pages run on the indices ("Show Me The Code", the quick
 * test): for query i, head h, over the valid entries c of idx[i, h, :]
 * (0 <= c < S; -1 and anything else is padding),
 *   w_c = exp(scale * q_i . k_c) / sum_c' exp(scale * q_i . k_c'),
 *   out[i, h, :] = sum_c w_c * v_c,
 * in double (the exponent is shifted by the row maximum, which leaves the
 * quotient unchanged), rounded once to float. A row without a valid entry
 * is zero. Repeated entries count once each, as in the pages' loop. */
static int attention_row(const void *q, const void *k, const void *v, int dt, int64_t S,
                         int32_t H, int32_t D, const int32_t *row, int32_t top_k,
                         double scale, int64_t i, int32_t h, double *s, double *acc,
                         float *o);

int oracle_sparse_attention(const void *q, const void *k, const void *v, int dt,
                            int64_t S, int32_t H, int32_t D, const int32_t *idx,
                            int32_t top_k, double scale, float *out)
{
    if (!q || !k || !v || !idx || !out || S < 1 || H < 1 || D < 1 || top_k < 1)
        return OR_EINVAL;
    if (dt != OR_F32 && dt != OR_BF16)
        return OR_EINVAL;
    double *s = (double *)malloc(sizeof(double) * (size_t)top_k);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    if (!s || !acc) {
        free(s);
        free(acc);
        return OR_ENOMEM;
    }
    for (int64_t i = 0; i < S; ++i)
        for (int32_t h = 0; h < H; ++h)
            attention_row(q, k, v, dt, S, H, D, idx + ((size_t)i * H + h) * (size_t)top_k, top_k,
                          scale, i, h, s, acc, out + ((size_t)i * H + h) * (size_t)D);
    free(s);
    free(acc);
    return OR_OK;
}

/* Selected rows: row r is query rows_i[r], head rows_h[r], with its index
 * row idx_rows[r, :]; out is (n_rows, D). */
int oracle_sparse_attention_rows(const void *q, const void *k, const void *v, int dt,
                                 int64_t S, int32_t H, int32_t D, const int32_t *idx_rows,
                                 int32_t top_k, int64_t n_rows, const int64_t *rows_i,
                                 const int32_t *rows_h, double scale, float *out)
{
    if (!q || !k || !v || !idx_rows || !rows_i || !rows_h || !out || S < 1 || H < 1 ||
        D < 1 || top_k < 1 || n_rows < 0)
        return OR_EINVAL;
    if (dt != OR_F32 && dt != OR_BF16)
        return OR_EINVAL;
    double *s = (double *)malloc(sizeof(double) * (size_t)top_k);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    if (!s || !acc) {
        free(s);
        free(acc);
        return OR_ENOMEM;
    }
    int rc = OR_OK;
    for (int64_t r = 0; r < n_rows; ++r) {
        if (rows_i[r] < 0 || rows_i[r] >= S || rows_h[r] < 0 || rows_h[r] >= H) {
            rc = OR_EINVAL;
            break;
        }
        attention_row(q, k, v, dt, S, H, D, idx_rows + (size_t)r * top_k, top_k, scale,
                      rows_i[r], rows_h[r], s, acc, out + (size_t)r * D);
    }
    free(s);
    free(acc);
    return rc;
}

/* One row of the attention: scores, shifted exponentials, weighted sum. */
static int attention_row(const void *q, const void *k, const void *v, int dt, int64_t S,
                         int32_t H, int32_t D, const int32_t *row, int32_t top_k,
                         double scale, int64_t i, int32_t h, double *s, double *acc,
                         float *o)
{
    double mx = -INFINITY;
    int any = 0;
    for (int t = 0; t < top_k; ++t) {
        int32_t c = row[t];
        s[t] = -INFINITY;
        if (c < 0 || c >= S)
            continue;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += (double)load_elem(q, dt, ((size_t)i * H + h) * D + d) *
                   (double)load_elem(k, dt, ((size_t)c * H + h) * D + d);
        s[t] = scale * dot;
        if (s[t] > mx)
            mx = s[t];
        any = 1;
    }
    for (int d = 0; d < D; ++d)
        acc[d] = 0.0;
    double den = 0.0;
    if (any) {
        for (int t = 0; t < top_k; ++t) {
            int32_t c = row[t];
            if (c < 0 || c >= S)
                continue;
            double e = exp(s[t] - mx);
            den += e;
            for (int d = 0; d < D; ++d)
                acc[d] += e * (double)load_elem(v, dt, ((size_t)c * H + h) * D + d);
        }
    }
    for (int d = 0; d < D; ++d)
        o[d] = any ? (float)(acc[d] / den) : 0.0f;
    return OR_OK;
}
