/*
 * Host-only driver for a sanitized build of the oracle (test
 * infrastructure): compiled together with oracle/pivot_oracle.c under
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitized.py, it calls every entry point on small
 * shapes (ragged last groups, g = 1, top_k beyond the prefix, both dtypes,
 * decode batches) and checks return codes and row structure. Any
 * out-of-bounds access, leak or undefined operation aborts the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_candidate_count(int32_t top_k, double candidate_ratio);
int oracle_proxy(const void *q, int dt, int64_t S, int32_t H, int32_t D, int32_t g, int32_t h, int64_t j,
                 float *out_p);
int oracle_prefill(const void *q, const void *k, int dt, int64_t S, int32_t H, int32_t D, int32_t top_k,
                   int32_t g, double candidate_ratio, int mode, int32_t h_begin, int32_t h_end,
                   int32_t *out_idx, float *out_score);
int oracle_prefill_rows(const void *q, const void *k, int dt, int64_t S, int32_t H, int32_t D, int32_t top_k,
                        int32_t g, double candidate_ratio, int mode, int64_t n_rows, const int64_t *rows_i,
                        const int32_t *rows_h, int32_t *out_idx, float *out_score);
int oracle_prefill_groups(const void *q, const void *k, int dt, int64_t S, int32_t H, int32_t D, int32_t top_k,
                          int32_t g, double candidate_ratio, int mode, int64_t n_groups, const int32_t *heads,
                          const int64_t *groups, int32_t *out_idx, float *out_score);
int64_t oracle_prefill_candidates(const void *q, const void *k, int dt, int64_t S, int32_t H, int32_t D,
                                  int32_t top_k, int32_t g, double candidate_ratio, int32_t h, int64_t j,
                                  int32_t *out_cand, float *out_score);
int oracle_dense(const void *q, const void *k, int dt, int64_t S, int32_t H, int32_t D, int32_t top_k,
                 int32_t h_begin, int32_t h_end, int32_t *out_idx, float *out_score);
int oracle_dense_rows(const void *q, const void *k, int dt, int64_t S, int32_t H, int32_t D, int32_t top_k,
                      int64_t n_rows, const int64_t *rows_i, const int32_t *rows_h, int32_t *out_idx,
                      float *out_score);
int oracle_decode(const void *q, const void *k_cache, int dt, const int64_t *ctx_lens, int32_t B, int32_t g,
                  int32_t H, int32_t D, int32_t top_k, double candidate_ratio, int mode, int32_t h_begin,
                  int32_t h_end, int32_t *out_idx, float *out_score);
int64_t oracle_decode_candidates(const void *q, const void *k_cache, int dt, const int64_t *ctx_lens, int32_t B,
                                 int32_t g, int32_t H, int32_t D, int32_t top_k, double candidate_ratio,
                                 int32_t h, int32_t b, int32_t *out_cand, float *out_score);
int oracle_sparse_attention(const void *q, const void *k, const void *v, int dt, int64_t S, int32_t H, int32_t D,
                            const int32_t *idx, int32_t top_k, double scale, float *out);
int oracle_sparse_attention_rows(const void *q, const void *k, const void *v, int dt, int64_t S, int32_t H,
                                 int32_t D, const int32_t *idx_rows, int32_t top_k, int64_t n_rows,
                                 const int64_t *rows_i, const int32_t *rows_h, double scale, float *out);

static uint64_t lcg = 88172645463325252ull;

static double uniform(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg >> 11) * (1.0 / 9007199254740992.0);
}

/* n elements of dtype dt (0 f32, 1 bf16 bits), values small integers or
 * uniform reals in [-2, 2) */
static void *draw(size_t n, int dt, int integer)
{
    void *p = malloc(n * (dt ? 2 : 4));
    for (size_t i = 0; i < n; ++i) {
        float x = integer ? (float)((int)(uniform() * 9.0) - 4) : (float)(uniform() * 4.0 - 2.0);
        if (dt) {
            uint32_t u;
            memcpy(&u, &x, 4);
            ((uint16_t *)p)[i] = (uint16_t)(u >> 16);
        } else {
            ((float *)p)[i] = x;
        }
    }
    return p;
}

static int fails = 0;

#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            fprintf(stderr, __VA_ARGS__);         \
            fputc('\n', stderr);                  \
            ++fails;                              \
        }                                         \
    } while (0)

/* rows of width top_k: valid entries (< limit, distinct) first, then -1 */
static void check_rows(const int32_t *idx, int64_t rows, int top_k, const int64_t *limit, const char *what)
{
    for (int64_t r = 0; r < rows; ++r) {
        const int32_t *row = idx + r * top_k;
        int t = 0;
        while (t < top_k && row[t] >= 0) {
            CHECK(row[t] < limit[r], "%s: row %lld slot %d index %d >= limit %lld", what, (long long)r, t,
                  row[t], (long long)limit[r]);
            for (int u = 0; u < t; ++u)
                CHECK(row[u] != row[t], "%s: row %lld duplicate", what, (long long)r);
            ++t;
        }
        for (; t < top_k; ++t)
            CHECK(row[t] == -1, "%s: row %lld slot %d not padding", what, (long long)r, t);
    }
}

static void prefill_case(int64_t S, int H, int D, int top_k, int g, double ratio, int dt, int integer)
{
    void *q = draw((size_t)S * H * D, dt, integer);
    void *k = draw((size_t)S * H * D, dt, integer);
    void *v = draw((size_t)S * H * D, dt, integer);
    size_t n = (size_t)S * H * top_k;
    int32_t *idx = malloc(n * 4);
    float *sc = malloc(n * 4);
    int64_t *lim = malloc(sizeof(int64_t) * (size_t)S * H);
    for (int mode = 0; mode < 3; ++mode) {
        CHECK(oracle_prefill(q, k, dt, S, H, D, top_k, g, ratio, mode, 0, H, idx, sc) == 0, "prefill rc");
        for (int64_t i = 0; i < S; ++i)
            for (int h = 0; h < H; ++h) {
                int64_t gs = (i / g) * g;
                lim[i * H + h] = mode == 2 ? (i > 0 ? i : 1) : (gs > 1 ? gs : 1);
            }
        check_rows(idx, S * H, top_k, lim, "prefill");
    }
    CHECK(oracle_dense(q, k, dt, S, H, D, top_k, 0, H, idx, sc) == 0, "dense rc");
    for (int64_t i = 0; i < S * H; ++i)
        lim[i] = (i / H) > 1 ? i / H : 1;
    check_rows(idx, S * H, top_k, lim, "dense");
    float *att = malloc(sizeof(float) * (size_t)S * H * D);
    CHECK(oracle_sparse_attention(q, k, v, dt, S, H, D, idx, top_k, 1.0 / sqrt((double)D), att) == 0,
          "attention rc");
    for (size_t i = 0; i < (size_t)S * H * D; ++i)
        CHECK(isfinite(att[i]), "attention output not finite");

    int64_t ri[4] = {0, S > 1 ? 1 : 0, S / 2, S - 1};
    int32_t rh[4] = {0, H - 1, 0, H - 1};
    int64_t rl[4];
    int32_t ridx[4 * 64];
    float rsc[4 * 64];
    if (top_k <= 64) {
        for (int mode = 0; mode < 3; ++mode) {
            CHECK(oracle_prefill_rows(q, k, dt, S, H, D, top_k, g, ratio, mode, 4, ri, rh, ridx, rsc) == 0,
                  "rows rc");
            for (int r = 0; r < 4; ++r) {
                int64_t gs = (ri[r] / g) * g;
                rl[r] = mode == 2 ? (ri[r] > 0 ? ri[r] : 1) : (gs > 1 ? gs : 1);
            }
            check_rows(ridx, 4, top_k, rl, "prefill rows");
        }
        CHECK(oracle_dense_rows(q, k, dt, S, H, D, top_k, 4, ri, rh, ridx, rsc) == 0, "dense rows rc");
        float arow[4 * 256];
        if (D <= 256)
            CHECK(oracle_sparse_attention_rows(q, k, v, dt, S, H, D, ridx, top_k, 4, ri, rh, 0.125, arow) == 0,
                  "attention rows rc");
    }
    int64_t G = (S + g - 1) / g;
    int32_t heads[2] = {0, H - 1};
    int64_t groups[2] = {0, G - 1};
    int32_t *gidx = malloc(sizeof(int32_t) * 2 * (size_t)g * top_k);
    float *gsc = malloc(sizeof(float) * 2 * (size_t)g * top_k);
    for (int mode = 0; mode < 2; ++mode)
        CHECK(oracle_prefill_groups(q, k, dt, S, H, D, top_k, g, ratio, mode, 2, heads, groups, gidx, gsc) == 0,
              "groups rc");
    int64_t K = oracle_candidate_count(top_k, ratio);
    int32_t *cand = malloc(sizeof(int32_t) * (size_t)K);
    float *csc = malloc(sizeof(float) * (size_t)K);
    int64_t nc = oracle_prefill_candidates(q, k, dt, S, H, D, top_k, g, ratio, H - 1, G - 1, cand, csc);
    CHECK(nc >= 1 && nc <= K, "candidates count %lld", (long long)nc);
    float *p = malloc(sizeof(float) * (size_t)D);
    CHECK(oracle_proxy(q, dt, S, H, D, g, 0, G - 1, p) == 0, "proxy rc");
    free(q), free(k), free(v), free(idx), free(sc), free(lim), free(att), free(gidx), free(gsc), free(cand),
        free(csc), free(p);
}

static void decode_case(int B, const int64_t *ctx, int g, int H, int D, int top_k, double ratio, int dt)
{
    int64_t total = 0;
    for (int b = 0; b < B; ++b)
        total += ctx[b];
    void *q = draw((size_t)B * g * H * D, dt, 1);
    void *kc = draw((size_t)total * H * D, dt, 1);
    size_t n = (size_t)B * g * H * top_k;
    int32_t *idx = malloc(n * 4);
    float *sc = malloc(n * 4);
    int64_t *lim = malloc(sizeof(int64_t) * (size_t)B * g * H);
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < g * H; ++t)
            lim[(int64_t)b * g * H + t] = ctx[b];
    for (int mode = 0; mode < 2; ++mode) {
        CHECK(oracle_decode(q, kc, dt, ctx, B, g, H, D, top_k, ratio, mode, 0, H, idx, sc) == 0, "decode rc");
        check_rows(idx, (int64_t)B * g * H, top_k, lim, "decode");
    }
    int64_t K = oracle_candidate_count(top_k, ratio);
    int32_t *cand = malloc(sizeof(int32_t) * (size_t)K);
    for (int b = 0; b < B; ++b) {
        int64_t nc = oracle_decode_candidates(q, kc, dt, ctx, B, g, H, D, top_k, ratio, H - 1, b, cand, NULL);
        CHECK(nc == (K < ctx[b] ? K : ctx[b]), "decode candidates count");
    }
    free(q), free(kc), free(idx), free(sc), free(lim), free(cand);
}

int main(void)
{
    prefill_case(37, 2, 16, 5, 8, 2.0, 0, 0);   /* ragged last group, fp32 */
    prefill_case(40, 3, 8, 7, 3, 1.5, 1, 1);    /* non-power-of-two groups, bf16 integers */
    prefill_case(21, 1, 8, 4, 1, 2.0, 1, 0);    /* g = 1 */
    prefill_case(12, 2, 4, 16, 16, 3.0, 0, 1);  /* top_k and g beyond S */
    prefill_case(1, 1, 4, 3, 2, 2.0, 1, 0);     /* a single position */
    int64_t ctx1[3] = {9, 1, 30};
    decode_case(3, ctx1, 2, 2, 8, 4, 2.0, 1);
    int64_t ctx2[2] = {5, 70};
    decode_case(2, ctx2, 4, 1, 16, 8, 1.0, 0);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("sanitized oracle run: all checks passed\n");
    return 0;
}
