/*
 * Drives the fp64 oracle (oracle/mla_oracle.c, linked in) under AddressSanitizer
 * and UndefinedBehaviorSanitizer: small paged caches of each kind (bf16, int8,
 * fp8), several threads, the plain and the split form, tokens subsets.  Exits
 * non-zero on a wrong result; the sanitizers abort on any memory error or
 * undefined behaviour.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int mla_oracle_attention(const uint16_t *q, int kv_kind, const void *cache, const float *kv_scale,
                         int num_pages, const int32_t *page_table, int max_pages, int page_size,
                         const int32_t *q_start, const int32_t *kv_len, int batch, int H, int dqk,
                         int dv, double softmax_scale, const int32_t *tokens, int ntokens,
                         double *out, double *lse, int nthreads);
int mla_oracle_attention_split(const uint16_t *q, int kv_kind, const void *cache,
                               const float *kv_scale, int num_pages, const int32_t *page_table,
                               int max_pages, int page_size, const int32_t *q_start,
                               const int32_t *kv_len, int batch, int H, int dqk, int dv,
                               double softmax_scale, const int32_t *bounds, int nranges,
                               const int32_t *tokens, int ntokens, double *out, double *lse,
                               int nthreads);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }
static float unit(void) { return (float)(next() & 0xFFFF) / 32768.0f - 1.0f; }
static uint16_t bf16(float x) { uint32_t u; memcpy(&u, &x, 4); return (uint16_t)(u >> 16); }

static int run_case(int kind, int page_size, int nthreads) {
    const int batch = 3, H = 4, dqk = 40, dv = 32;
    const int kv_len[3] = {70, 1, 130};
    const int q_len[3] = {2, 1, 5};
    int32_t q_start[4] = {0, 0, 0, 0}, lens[3];
    for (int b = 0; b < batch; ++b) { q_start[b + 1] = q_start[b] + q_len[b]; lens[b] = kv_len[b]; }
    const int T = q_start[batch];
    const int max_pages = (130 + page_size - 1) / page_size;
    int num_pages = 0;
    for (int b = 0; b < batch; ++b) num_pages += (kv_len[b] + page_size - 1) / page_size;
    int32_t *pt = malloc(sizeof(int32_t) * batch * max_pages);
    int p = num_pages - 1;
    for (int b = 0; b < batch; ++b)
        for (int j = 0; j < max_pages; ++j)
            pt[b * max_pages + j] = j < (kv_len[b] + page_size - 1) / page_size ? p-- : 0;
    const size_t rows = (size_t)num_pages * page_size;
    void *cache;
    float *scale = NULL;
    if (kind == 0) {
        uint16_t *c = malloc(rows * dqk * 2);
        for (size_t i = 0; i < rows * dqk; ++i) c[i] = bf16(unit());
        cache = c;
    } else {
        uint8_t *c = malloc(rows * dqk);
        for (size_t i = 0; i < rows * dqk; ++i) {
            uint8_t v = (uint8_t)(next() & 0xFF);
            if (kind == 1 && v == 0x80) v = 0x81;             /* int8: codes -127 .. 127 */
            if (kind == 2 && (v & 0x7F) == 0x7F) v ^= 1;     /* E4M3: no NaN codes */
            c[i] = v;
        }
        cache = c;
        scale = malloc(rows * sizeof(float));
        for (size_t i = 0; i < rows; ++i) scale[i] = 0.01f + 0.001f * (float)(i % 7);
    }
    uint16_t *q = malloc((size_t)T * H * dqk * 2);
    for (size_t i = 0; i < (size_t)T * H * dqk; ++i) q[i] = bf16(unit());
    double *o1 = malloc(sizeof(double) * T * H * dv), *l1 = malloc(sizeof(double) * T * H);
    double *o2 = malloc(sizeof(double) * T * H * dv), *l2 = malloc(sizeof(double) * T * H);
    const double sc = 1.0 / sqrt(192.0);
    int rc = mla_oracle_attention(q, kind, cache, scale, num_pages, pt, max_pages, page_size, q_start, lens, batch,
                                  H, dqk, dv, sc, NULL, 0, o1, l1, nthreads);
    if (rc) { fprintf(stderr, "attention rc %d\n", rc); return 1; }
    const int32_t bounds[4] = {0, 17, 64, 200};
    rc = mla_oracle_attention_split(q, kind, cache, scale, num_pages, pt, max_pages, page_size, q_start, lens,
                                    batch, H, dqk, dv, sc, bounds, 3, NULL, 0, o2, l2, nthreads);
    if (rc) { fprintf(stderr, "split rc %d\n", rc); return 1; }
    for (int i = 0; i < T * H; ++i) {
        if (!isfinite(l1[i]) || fabs(l1[i] - l2[i]) > 1e-12 * (1 + fabs(l1[i]))) {
            fprintf(stderr, "lse mismatch at %d: %g %g\n", i, l1[i], l2[i]);
            return 1;
        }
        for (int d = 0; d < dv; ++d)
            if (fabs(o1[i * dv + d] - o2[i * dv + d]) > 1e-12 * (1 + fabs(o1[i * dv + d]))) {
                fprintf(stderr, "out mismatch at %d,%d\n", i, d);
                return 1;
            }
    }
    const int32_t toks[2] = {T - 1, 0};
    rc = mla_oracle_attention(q, kind, cache, scale, num_pages, pt, max_pages, page_size, q_start, lens, batch, H,
                              dqk, dv, sc, toks, 2, o2, l2, nthreads);
    if (rc || l2[0] != l1[(T - 1) * H] || l2[H] != l1[0]) { fprintf(stderr, "token subset mismatch\n"); return 1; }
    free(pt); free(cache); free(scale); free(q); free(o1); free(l1); free(o2); free(l2);
    return 0;
}

int main(void) {
    for (int kind = 0; kind < 3; ++kind)
        for (int ps = 16; ps <= 64; ps *= 4)
            for (int nt = 1; nt <= 3; nt += 2)
                if (run_case(kind, ps, nt)) { fprintf(stderr, "kind %d page %d threads %d\n", kind, ps, nt); return 1; }
    puts("oracle driver ok");
    return 0;
}
