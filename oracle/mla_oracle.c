/*
 * Plain fp64 CPU oracle for Multi-head Latent Attention (MLA) over a paged,
 * compressed latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent definition that
 * the HIP path is checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the library's compute path
 * never calls it and shares no code, header or table with it.
 *
 * Sources (web pages on the TokenSpeed inference engine):
 *   [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎" -- AICon 2026 Shenzhen
 *          talk transcript, sections "Kernel：让 MLA 真正跑满 GPU" and
 *          "跨平台 Kernel 设计".
 *   [NEWS] "英偉達力薦，小團隊兩個月開源一款「光速級」智能體推理引擎" -- news
 *          article, sections "TokenSpeed 技術簡介" and "TokenSpeed 性能預覽".
 *   [MLA]  The published MLA formulation (DeepSeek-V2, arXiv:2405.04434),
 *          used only for the absorbed form and the 192-wide score scale.
 *   [GITREAD] "TokenSpeed 深度解析:把 LLM 推理压到"光速"意味着什么" --
 *          third-party project commentary, section "核心技术揭秘".
 *
 * What is computed (the plain definition; every kernel technique on the
 * pages -- folding the query axis into the heads, split-KV, paging, online
 * softmax -- is an exact reformulation of it):
 *
 *   [TALK, "Kernel：让 MLA 真正跑满 GPU"]: the KV of all heads is one
 *   compressed latent row per token, and the first product of decode
 *   attention is query x latent key.  Read in absorbed form [MLA]: the key
 *   of token t is its whole cache row c_t (latent 0..dv-1, rope dv..dqk-1),
 *   the value is its first dv columns, and all H query heads attend the
 *   same rows.
 *
 *   Request b holds kv_len[b] rows; its n_b query tokens are the last n_b of
 *   them (decode: n_b = q_len, speculative drafts causal among themselves
 *   [NEWS, "TokenSpeed 性能預覽"]; prefill: the appended tokens after a
 *   cached prefix, different Q and KV lengths, no padding [TALK,
 *   "Kernel：让 MLA 真正跑满 GPU"]).  Query token i (0-based) sees rows
 *   0 .. kv_len[b] - n_b + i.
 *
 *     s_t   = softmax_scale * sum_{d < dqk} q[d] * c_t[d]
 *     lse   = m + ln sum_t exp(s_t - m),  m = max_t s_t      (natural log)
 *     out_d = sum_t exp(s_t - lse) * c_t[d],  d < dv
 *
 *   Row gather: c_t = cache[page_table[b][t / page_size]][t % page_size];
 *   for the INT8 cache c_t[d] = code * scale[page][slot]; for the FP8 cache
 *   c_t[d] = e4m3(code) * scale[page][slot].
 *
 *   FP8 [GITREAD] "TokenSpeed 深度解析:把 LLM 推理压到"光速"意味着什么",
 *   section "核心技术揭秘": FP8 KV-cache quantisation is named as standard,
 *   with no format given.  Read here as the 8-bit "E4M3" format of the OCP
 *   8-bit floating point specification (finite variant): sign bit 7,
 *   exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 encodes
 *   the subnormals m * 2^-9; the all-ones magnitude 0x7F is NaN; there is no
 *   infinity, so the largest finite magnitude is 448.  Each row carries an
 *   fp32 scale as the INT8 cache does.
 *
 *   Split form [TALK, "Kernel：让 MLA 真正跑满 GPU": phase one computes
 *   split-KV partial results, phase two reduces them]: for a partition of
 *   the visible rows into ranges R_k, lse_k and o_k are the above over R_k
 *   alone (lse_k = -inf and o_k = 0 for an empty range); then
 *   lse = ln sum_k exp(lse_k) and out = sum_k exp(lse_k - lse) * o_k.
 *
 * Inputs are read exactly as the GPU receives them (bf16 bit patterns, int8
 * or fp8 codes with fp32 scales) and widened exactly to double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_OK = 0, ORACLE_EINVAL = 1 };

typedef struct {
    const uint16_t *q;
    int kv_kind; /* 0: bf16 rows, 1: int8 codes, 2: fp8 e4m3 codes; 1, 2: + fp32 per-row scale */
    const void *cache;
    const float *kv_scale;
    int num_pages;
    const int32_t *page_table;
    int max_pages;
    int page_size;
    const int32_t *q_start;
    const int32_t *kv_len;
    int batch, H, dqk, dv;
    double softmax_scale;
    const int32_t *tokens; /* query tokens to evaluate, or NULL for 0..total-1 */
    int ntokens;
    const int32_t *bounds; /* split form: nranges+1 ascending row positions, or NULL */
    int nranges;
    double *out;
    double *lse;
    int next_row;          /* shared work counter */
    int error;
} job_t;

static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Value of an E4M3 code, from the format's definition (see the header). */
double mla_oracle_e4m3_value(uint8_t code)
{
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Request that owns global query token tok: q_start[b] <= tok < q_start[b+1]. */
static int owner_of(const job_t *j, int tok)
{
    for (int b = 0; b < j->batch; ++b)
        if (tok >= j->q_start[b] && tok < j->q_start[b + 1]) return b;
    return -1;
}

/* Row gather: the dqk values of row t of request b, widened to double. */
static int gather_row(const job_t *j, int b, int t, double *c)
{
    int pj = t / j->page_size, slot = t % j->page_size;
    if (pj < 0 || pj >= j->max_pages) return ORACLE_EINVAL;
    int page = j->page_table[(size_t)b * j->max_pages + pj];
    if (page < 0 || page >= j->num_pages) return ORACLE_EINVAL;
    size_t base = ((size_t)page * j->page_size + slot) * j->dqk;
    if (j->kv_kind == 0) {
        const uint16_t *row = (const uint16_t *)j->cache + base;
        for (int d = 0; d < j->dqk; ++d) c[d] = bf16_to_double(row[d]);
    } else if (j->kv_kind == 1) {
        const int8_t *row = (const int8_t *)j->cache + base;
        double s = (double)j->kv_scale[(size_t)page * j->page_size + slot];
        for (int d = 0; d < j->dqk; ++d) c[d] = (double)row[d] * s;
    } else {
        const uint8_t *row = (const uint8_t *)j->cache + base;
        double s = (double)j->kv_scale[(size_t)page * j->page_size + slot];
        for (int d = 0; d < j->dqk; ++d) c[d] = mla_oracle_e4m3_value(row[d]) * s;
    }
    return ORACLE_OK;
}

/* Attention of one (query token, head) row over visible rows [lo, hi).
 * Writes o[0..dv) and returns lse; an empty range gives lse = -inf, o = 0. */
static int attend_range(const job_t *j, int b, const double *qd, int lo, int hi,
                        double *s, double *c, double *o, double *lse_out)
{
    for (int d = 0; d < j->dv; ++d) o[d] = 0.0;
    if (hi <= lo) {
        *lse_out = -INFINITY;
        return ORACLE_OK;
    }
    /* scores */
    for (int t = lo; t < hi; ++t) {
        if (gather_row(j, b, t, c)) return ORACLE_EINVAL;
        double acc = 0.0;
        for (int d = 0; d < j->dqk; ++d) acc += qd[d] * c[d];
        s[t - lo] = j->softmax_scale * acc;
    }
    /* log-sum-exp */
    double m = -INFINITY;
    for (int t = lo; t < hi; ++t)
        if (s[t - lo] > m) m = s[t - lo];
    double sum = 0.0;
    for (int t = lo; t < hi; ++t) sum += exp(s[t - lo] - m);
    double lse = m + log(sum);
    /* probability-weighted sum of the value columns */
    for (int t = lo; t < hi; ++t) {
        if (gather_row(j, b, t, c)) return ORACLE_EINVAL;
        double w = exp(s[t - lo] - lse);
        for (int d = 0; d < j->dv; ++d) o[d] += w * c[d];
    }
    *lse_out = lse;
    return ORACLE_OK;
}

static int do_row(job_t *j, int row, double *s, double *c, double *qd, double *part_o,
                  double *part_lse)
{
    int idx = row / j->H, h = row % j->H;
    int tok = j->tokens ? j->tokens[idx] : idx;
    int b = owner_of(j, tok);
    if (b < 0) return ORACLE_EINVAL;
    int n_b = j->q_start[b + 1] - j->q_start[b];
    int i = tok - j->q_start[b];
    int L = j->kv_len[b];
    int last = L - n_b + i; /* bottom-right aligned causal limit */
    if (n_b > L || last < 0 || last >= L) return ORACLE_EINVAL;

    const uint16_t *qr = j->q + ((size_t)tok * j->H + h) * j->dqk;
    for (int d = 0; d < j->dqk; ++d) qd[d] = bf16_to_double(qr[d]);

    double *out = j->out + (size_t)row * j->dv;
    double *lse = j->lse + row;

    if (!j->bounds) return attend_range(j, b, qd, 0, last + 1, s, c, out, lse);

    /* split form: partials over each range intersected with the visible set */
    for (int k = 0; k < j->nranges; ++k) {
        int lo = j->bounds[k], hi = j->bounds[k + 1];
        if (hi > last + 1) hi = last + 1;
        if (lo < 0) lo = 0;
        if (attend_range(j, b, qd, lo, hi, s, c, part_o + (size_t)k * j->dv, part_lse + k))
            return ORACLE_EINVAL;
    }
    /* merge: lse = ln sum_k exp(lse_k); out = sum_k exp(lse_k - lse) o_k */
    double m = -INFINITY;
    for (int k = 0; k < j->nranges; ++k)
        if (part_lse[k] > m) m = part_lse[k];
    double sum = 0.0;
    for (int k = 0; k < j->nranges; ++k)
        if (part_lse[k] != -INFINITY) sum += exp(part_lse[k] - m);
    double total = m + log(sum);
    for (int d = 0; d < j->dv; ++d) out[d] = 0.0;
    for (int k = 0; k < j->nranges; ++k) {
        if (part_lse[k] == -INFINITY) continue;
        double w = exp(part_lse[k] - total);
        for (int d = 0; d < j->dv; ++d) out[d] += w * part_o[(size_t)k * j->dv + d];
    }
    *lse = total;
    return ORACLE_OK;
}

static void *worker(void *arg)
{
    job_t *j = (job_t *)arg;
    int maxlen = 0;
    for (int b = 0; b < j->batch; ++b)
        if (j->kv_len[b] > maxlen) maxlen = j->kv_len[b];
    double *s = malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
    double *c = malloc(sizeof(double) * (size_t)j->dqk);
    double *qd = malloc(sizeof(double) * (size_t)j->dqk);
    int nr = j->bounds ? j->nranges : 1;
    double *po = malloc(sizeof(double) * (size_t)nr * j->dv);
    double *pl = malloc(sizeof(double) * (size_t)nr);
    if (!s || !c || !qd || !po || !pl) {
        __atomic_store_n(&j->error, ORACLE_EINVAL, __ATOMIC_RELAXED);
    } else {
        int rows = j->ntokens * j->H;
        for (;;) {
            int row = __atomic_fetch_add(&j->next_row, 1, __ATOMIC_RELAXED);
            if (row >= rows) break;
            if (do_row(j, row, s, c, qd, po, pl))
                __atomic_store_n(&j->error, ORACLE_EINVAL, __ATOMIC_RELAXED);
        }
    }
    free(s);
    free(c);
    free(qd);
    free(po);
    free(pl);
    return NULL;
}

static int run(job_t *j, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int k = 0; k < nthreads; ++k) {
        if (pthread_create(&th[k], NULL, worker, j) != 0) break;
        ++started;
    }
    if (started == 0) worker(j);
    for (int k = 0; k < started; ++k) pthread_join(th[k], NULL);
    return j->error;
}

static int check_common(const job_t *j)
{
    if (!j->q || !j->cache || !j->page_table || !j->q_start || !j->kv_len || !j->out || !j->lse)
        return ORACLE_EINVAL;
    if (j->kv_kind != 0 && !j->kv_scale) return ORACLE_EINVAL;
    if (j->kv_kind < 0 || j->kv_kind > 2) return ORACLE_EINVAL;
    if (j->batch < 1 || j->H < 1 || j->dqk < 1 || j->dv < 1 || j->dv > j->dqk || j->page_size < 1)
        return ORACLE_EINVAL;
    if (j->ntokens < 0) return ORACLE_EINVAL;
    return ORACLE_OK;
}

/*
 * Attention for the query tokens listed in `tokens` (global indices into q;
 * NULL means all q_start[batch] tokens), all heads.  out is
 * [ntokens, H, dv], lse is [ntokens, H] (natural log).  Returns 0, or 1 on
 * an invalid argument or an out-of-range page reference.
 */
int mla_oracle_attention(const uint16_t *q, int kv_kind, const void *cache, const float *kv_scale,
                         int num_pages, const int32_t *page_table, int max_pages, int page_size,
                         const int32_t *q_start, const int32_t *kv_len, int batch, int H, int dqk,
                         int dv, double softmax_scale, const int32_t *tokens, int ntokens,
                         double *out, double *lse, int nthreads)
{
    job_t j = {q, kv_kind, cache, kv_scale, num_pages, page_table, max_pages, page_size,
               q_start, kv_len, batch, H, dqk, dv, softmax_scale, tokens,
               tokens ? ntokens : (q_start ? q_start[batch] : 0), NULL, 0, out, lse, 0, 0};
    if (check_common(&j)) return ORACLE_EINVAL;
    return run(&j, nthreads);
}

/*
 * The split form: the visible rows of every (token, head) are partitioned
 * by the ranges [bounds[k], bounds[k+1]), k < nranges, each range reduced
 * to (lse_k, o_k) on its own and the partials merged.  bounds must start at
 * 0, be non-decreasing and end at or past every request's length.
 */
int mla_oracle_attention_split(const uint16_t *q, int kv_kind, const void *cache,
                               const float *kv_scale, int num_pages, const int32_t *page_table,
                               int max_pages, int page_size, const int32_t *q_start,
                               const int32_t *kv_len, int batch, int H, int dqk, int dv,
                               double softmax_scale, const int32_t *bounds, int nranges,
                               const int32_t *tokens, int ntokens, double *out, double *lse,
                               int nthreads)
{
    job_t j = {q, kv_kind, cache, kv_scale, num_pages, page_table, max_pages, page_size,
               q_start, kv_len, batch, H, dqk, dv, softmax_scale, tokens,
               tokens ? ntokens : (q_start ? q_start[batch] : 0), bounds, nranges, out, lse, 0, 0};
    if (check_common(&j) || !bounds || nranges < 1 || bounds[0] != 0) return ORACLE_EINVAL;
    for (int k = 0; k < nranges; ++k)
        if (bounds[k + 1] < bounds[k]) return ORACLE_EINVAL;
    for (int b = 0; b < batch; ++b)
        if (bounds[nranges] < kv_len[b]) return ORACLE_EINVAL;
    return run(&j, nthreads);
}
