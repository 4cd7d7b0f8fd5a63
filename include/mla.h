/*
 * mla.h -- C ABI of a gfx950 (MI355X) library for Multi-head Latent
 * Attention (MLA) over a paged, compressed latent KV cache.
 *
 * Sources (web pages on the TokenSpeed inference engine):
 *   [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎" -- AICon 2026 Shenzhen
 *          talk transcript.
 *   [NEWS] "英偉達力薦，小團隊兩個月開源一款「光速級」智能體推理引擎" -- news
 *          article on the TokenSpeed blog post.
 *   [GITREAD] "TokenSpeed 深度解析:把 LLM 推理压到"光速"意味着什么" --
 *          third-party commentary on the project.
 *
 * What is computed.  [TALK, section "Kernel：让 MLA 真正跑满 GPU"]: MLA keeps
 * the KV of every head as one compressed latent row per token, and the first
 * product of decode attention is query x latent key.  Here (absorbed form)
 * a cache row is 576 bf16 values, the 512 latent columns followed by the 64
 * rope columns; the key of a token is its whole row and its value is the
 * first 512 columns of that same row; all query heads attend the same rows.
 * For a query row q (576 values) of request b and the rows t it sees:
 *
 *     s_t  = softmax_scale * <q, row_t>
 *     lse  = ln sum_t exp(s_t)                       (natural log, fp32)
 *     out  = sum_t exp(s_t - lse) * row_t[0:512]     (bf16, rounded to nearest even)
 *
 * Causality: a request with L cached rows and n new query tokens (the last
 * n of its L rows) lets new token i (0-based) see rows 0 .. L-n+i.  That
 * covers speculative-decoding verification, where the drafts are causal
 * among themselves [NEWS, section "TokenSpeed 性能預覽"], and prefill after
 * a cached prefix, where Q and KV lengths differ [TALK, section
 * "Kernel：让 MLA 真正跑满 GPU"].
 *
 * Memory layouts (all device memory, all row-major, no padding):
 *   query      bf16 [tokens, num_heads, 576]
 *   kv_cache   bf16, int8 or fp8 [num_pages, page_size, 576]; page_size is
 *              a multiple of 64 up to MLA_MAX_PAGE_SIZE
 *   kv_scale   fp32 [num_pages, page_size]: per-row scale of the int8 and
 *              fp8 caches (row value = code * scale, or e4m3(code) * scale);
 *              NULL for a bf16 cache
 *   page_table int32 [batch, max_pages_per_req]: physical page of logical
 *              page j of request b (rows j * page_size ..); only entries
 *              j < ceil(L_b / page_size) are read
 *   out        bf16 [tokens, num_heads, 512]
 *   lse        fp32 [tokens, num_heads]
 *
 * FP8 cache [GITREAD] "TokenSpeed 深度解析:把 LLM 推理压到"光速"意味着什么",
 * section "核心技术揭秘" (FP8 KV-cache quantisation, no format given): codes
 * are OCP E4M3, finite variant -- sign bit 7, exponent bits 6..3 with bias
 * 7, mantissa bits 2..0, subnormals m * 2^-9, largest magnitude 448; the
 * magnitude 0x7F (NaN) must not occur in a cache.  Codes are widened to
 * bf16 exactly; attention then runs as for bf16 with the row scales applied
 * to the scores and probabilities.
 *
 * Page sizes [TALK, section "Runtime：构建可扩展的推理引擎架构": the engine's
 * first cache managed blocks of 1536 tokens; its later two-level design has
 * logical blocks of 128 tokens, for finer prefix reuse, inside physical
 * blocks of 1536].  A page of page_size rows is, in memory, page_size / 64
 * consecutive 64-row sub-pages, which is how the kernels walk it.  The
 * two-level layout is page_size = 128 with each entry naming the 128-row
 * block (physical block * 12 + slot) that holds the logical block; one-level
 * 1536-row blocks are page_size = 1536.
 *
 * Ownership and streams.  The caller allocates every buffer; the library
 * never allocates or frees device memory, never synchronises, keeps no
 * pointer after a call returns, and enqueues all work on `hip_stream`
 * (a hipStream_t; NULL is the default stream).  Buffers must stay valid
 * until that work has finished.  The workspace is scratch owned by the call
 * while it runs; calls that share one workspace must be ordered on one stream.
 *
 * Errors.  Every function returns an MLA_STATUS code.  Host-side scalar
 * arguments are all checked before any HIP call, so invalid arguments are
 * reported on a machine without a GPU.  Device-resident lengths are
 * preconditions, not checked: q_len <= seq_lens[b] <= max_seq_len (decode),
 * new tokens + prefix_lens[b] <= max_seq_len (prefill), and the page-table
 * entries that are read name pages that exist.  Lengths above
 * max_pages_per_req * page_size are clamped on the device so that the page table is
 * never read out of bounds.
 *
 * Determinism.  For fixed inputs and shapes the results are bitwise
 * reproducible, and bitwise invariant under a permutation of the physical
 * pages.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID 1     /* null pointer, non-positive size, inconsistent sizes */
#define MLA_ERR_UNSUPPORTED 2 /* valid but not implemented: page size, row count, dtype */
#define MLA_ERR_WORKSPACE 3   /* workspace smaller than mla_splitkv_workspace_size() */
#define MLA_ERR_HIP 4         /* a HIP runtime call or kernel launch failed */
#define MLA_ERR_SCRATCH 5     /* mla_decode_noalloc: the split-KV workspace the shape needs
                                 exceeds MLA_NOALLOC_SCRATCH_BYTES */

/* Cache element types. */
#define MLA_KV_BF16 0
#define MLA_KV_INT8 1
#define MLA_KV_FP8 2  /* E4M3 codes, see the layouts above */

#define MLA_DIM_QK 576      /* cache row / query row width: 512 latent + 64 rope */
#define MLA_DIM_V 512       /* value width: the first 512 columns of a row */
#define MLA_DIM_NOPE 128    /* per-head query / key width without position (unabsorbed) */
#define MLA_DIM_ROPE 64     /* per-head rotary part, shared by query and cache row */
#define MLA_DIM_VHEAD 128   /* per-head value width after the up-projection */
#define MLA_PAGE_SIZE 64    /* the kernels' sub-page: page sizes are multiples of it */
#define MLA_MAX_PAGE_SIZE 4096 /* largest page size */
#define MLA_MAX_DECODE_ROWS 128 /* q_len * num_heads of one decode request */
#define MLA_MAX_HEADS 128   /* prefill: heads of one query token */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20) /* fixed scratch of mla_decode_noalloc, per GPU */

/*
 * Workspace bytes for mla_decode, mla_decode_varlen and mla_prefill_varlen
 * [TALK, section "Kernel：让 MLA 真正跑满 GPU": the split parameters and the
 * workspace size are computed at run time and cached].
 *
 * One function serves every entry point.  For decode pass
 * max_q_len = q_len and total_q = batch * q_len; for the other two pass the
 * largest and the total number of query tokens.  The result is an upper bound
 * that depends only on these scalars and the current device's compute-unit
 * count, never on device-resident lengths, so a buffer sized once serves
 * every call with the same or smaller arguments.  It may be 0.
 *
 * Returns MLA_OK, MLA_ERR_INVALID (bytes_out NULL, batch, num_heads or
 * max_seq_len < 1, max_q_len or total_q < 0), MLA_ERR_UNSUPPORTED
 * (kv_dtype), or MLA_ERR_HIP when
 * the device cannot be queried.
 */
int mla_splitkv_workspace_size(int batch, int num_heads, int max_q_len, int total_q,
                               int max_seq_len, int kv_dtype, size_t* bytes_out);

/*
 * Decode: each of `batch` requests appends q_len query tokens (one new token
 * plus q_len - 1 speculative drafts, causal among themselves).
 *
 * The q_len tokens are folded into the head axis, so one request is a block
 * of q_len * num_heads query rows (row i * num_heads + h is head h of token
 * i) against one latent row per cached token [NEWS, section
 * "TokenSpeed 性能預覽": the decode kernel folds the query-sequence axis into
 * the head axis; TALK, section "Kernel：让 MLA 真正跑满 GPU": fold factor].
 * The cached rows are split across compute units and the partial results
 * (normalised output plus log-sum-exp) are reduced in a second phase [TALK,
 * same section: two-phase split-KV].
 *
 *   q          bf16 [batch * q_len, num_heads, 576]; token b * q_len + i is
 *              draft i of request b
 *   kv_cache, kv_scale, kv_dtype, page_table, max_pages_per_req: see above
 *   seq_lens   int32 [batch] on the device: cached rows of request b,
 *              the q_len new tokens included
 *   max_seq_len  host upper bound of seq_lens; max_pages_per_req must be
 *              at least ceil(max_seq_len / page_size).  The bf16 kernel also
 *              requests each workgroup's first tile before the lengths
 *              arrive, guessing that every request holds max_seq_len rows;
 *              the guess is checked, so any lengths give the same result,
 *              and batches whose lengths all equal max_seq_len start soonest
 *   softmax_scale  multiplies <q, row> (for example 1/sqrt(192))
 *   out, lse   outputs, [batch * q_len, num_heads, 512] bf16 and
 *              [batch * q_len, num_heads] fp32
 *   workspace  device scratch of at least mla_splitkv_workspace_size(batch,
 *              num_heads, q_len, batch * q_len, max_seq_len, kv_dtype)
 *              bytes, 256-byte aligned; may be NULL when that size is 0
 *
 * Returns MLA_OK; MLA_ERR_INVALID for a null pointer, a size < 1, a
 * non-finite or non-positive softmax_scale, max_seq_len < q_len or
 * max_pages_per_req too small; MLA_ERR_UNSUPPORTED for a page_size that is
 * not a multiple of 64 in 64 .. MLA_MAX_PAGE_SIZE,
 * q_len * num_heads > 128 or an unknown kv_dtype; MLA_ERR_WORKSPACE;
 * MLA_ERR_HIP.
 */
int mla_decode(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
               const int32_t* page_table, int max_pages_per_req, const int32_t* seq_lens,
               int batch, int q_len, int num_heads, int page_size, int max_seq_len,
               float softmax_scale, void* out, float* lse, void* workspace,
               size_t workspace_bytes, void* hip_stream);

/*
 * Decode with a different number of query tokens per request: speculative
 * decoding verifies a variable number of drafts per request [NEWS, section
 * "TokenSpeed 性能預覽": speculative decoding, drafts causal among
 * themselves].  Everything is as for mla_decode except the query layout:
 *
 *   q              bf16 [total_q, num_heads, 576], packed: request b's
 *                  tokens are cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1
 *   cu_seqlens_q   int32 [batch+1] on the device, cu_seqlens_q[0] = 0,
 *                  nondecreasing, n_b = cu_seqlens_q[b+1] - cu_seqlens_q[b]
 *                  <= max_q_len and n_b <= seq_lens[b] (preconditions)
 *   total_q        cu_seqlens_q[batch] (host), 0 <= total_q <= batch * max_q_len
 *   max_q_len      host upper bound of n_b; max_q_len * num_heads <= 128
 *   out, lse       [total_q, num_heads, 512] bf16 and [total_q, num_heads] fp32
 *   workspace      at least mla_splitkv_workspace_size(batch, num_heads,
 *                  max_q_len, total_q, max_seq_len, kv_dtype) bytes
 *
 * Token i of request b (0-based) sees rows 0 .. seq_lens[b] - n_b + i.  A
 * request with n_b = 0 produces nothing; total_q = 0 enqueues nothing (and
 * then only the scalar arguments are checked: pointers may be NULL).
 * Returns as mla_decode, plus MLA_ERR_INVALID for a null cu_seqlens_q or a
 * total_q outside 0 .. batch * max_q_len.
 */
int mla_decode_varlen(const void* q, const int32_t* cu_seqlens_q, const void* kv_cache, const float* kv_scale,
                      int kv_dtype, const int32_t* page_table, int max_pages_per_req, const int32_t* seq_lens,
                      int batch, int total_q, int max_q_len, int num_heads, int page_size, int max_seq_len,
                      float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* hip_stream);

/*
 * Variable-length prefill after a cached prefix, without padding
 * [TALK, section "Kernel：让 MLA 真正跑满 GPU": agent requests hit a cached
 * prefix and append a few hundred tokens, so Q and KV lengths differ and the
 * kernel batches variable lengths with no padding].  Work tiles of query
 * tokens are taken from a device-side queue by a persistent grid so that
 * uneven requests balance across compute units [TALK, section
 * "跨平台 Kernel 设计": a persistent prefill kernel balances scheduling on
 * MI355X].
 *
 *   q             bf16 [total_q, num_heads, 576], the new tokens of all
 *                 requests back to back
 *   cu_seqlens_q  int32 [batch + 1] on the device: request b owns tokens
 *                 cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; cu_seqlens_q[0] = 0,
 *                 cu_seqlens_q[batch] = total_q
 *   prefix_lens   int32 [batch] on the device: cached rows before the new
 *                 tokens; request b attends prefix_lens[b] + n_b rows, whose
 *                 last n_b rows must already hold the new tokens' latent rows
 *   max_q_len     host upper bound of the new-token counts
 *   max_seq_len   host upper bound of prefix_lens[b] + n_b
 *   other arguments as for mla_decode; out/lse are [total_q, num_heads, ...]
 *   workspace     at least mla_splitkv_workspace_size(batch, num_heads,
 *                 max_q_len, total_q, max_seq_len, kv_dtype) bytes
 *
 * A request with no new tokens writes nothing.  Returns as mla_decode;
 * num_heads > 128 is MLA_ERR_UNSUPPORTED; total_q = 0 returns MLA_OK
 * without launching.
 */
int mla_prefill_varlen(const void* q, const int32_t* cu_seqlens_q, const int32_t* prefix_lens,
                       const void* kv_cache, const float* kv_scale, int kv_dtype,
                       const int32_t* page_table, int max_pages_per_req, int batch, int total_q,
                       int max_q_len, int max_seq_len, int num_heads, int page_size,
                       float softmax_scale, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* hip_stream);

/*
 * mla_kv_append -- write the rows of new tokens into their requests' pages.
 *
 * The step that precedes attention: decode and prefill read a request's new
 * tokens from the cache [TALK, section "Kernel：让 MLA 真正跑满 GPU": the
 * attention kernels run over the paged latent cache, and at long prefixes
 * decode stays bandwidth-bound even with an INT8 latent cache].  For request
 * b, new row j (0 <= j < n_b = cu_seqlens_new[b+1] - cu_seqlens_new[b]) is
 * row cu_seqlens_new[b] + j of kv_new and goes to logical position
 * t = start_pos[b] + j of the request: page page_table[b][t / page_size],
 * slot t % page_size.
 *
 *   bf16 cache (kv_dtype 0): the 576 values are copied unchanged.
 *   int8 cache (kv_dtype 1): symmetric per-row quantisation with an fp32
 *     scale: scale = max_c |x_c| / 127 (fp32 division, rounded to nearest;
 *     an all-zero row gets scale 1), code_c = clamp(rint(x_c / scale),
 *     -127, 127) with ties to even; the codes go to the row of the int8 cache
 *     and the scale to kv_scale[page * page_size + slot].  Dequantised value:
 *     code * scale, as the attention entry points read it.
 *   fp8 cache (kv_dtype 2) [GITREAD, section "核心技术揭秘"]: the same with
 *     scale = max_c |x_c| / 448 and code_c = the E4M3 value nearest to
 *     x_c / scale (fp32 division), ties to the even mantissa, magnitudes
 *     above 448 saturating to 448.  Dequantised value: e4m3(code) * scale.
 *     Inputs must be finite.
 *
 *   kv_new          bf16 [total_new, 576] (latent | rope)
 *   cu_seqlens_new  int32 [batch+1], cu_seqlens_new[0] = 0, nondecreasing,
 *                   cu_seqlens_new[batch] = total_new
 *   start_pos       int32 [batch]: logical position of each request's first
 *                   new row (its cached length before the append)
 *   kv_cache        bf16, int8 or fp8 [num_pages, page_size, 576], written in place
 *   kv_scale        fp32 [num_pages, page_size] for an int8 or fp8 cache (written),
 *                   else NULL
 *   page_table      int32 [batch, max_pages_per_req]
 *
 * Rows whose position falls outside 0 .. max_pages_per_req * page_size - 1 are not
 * written.  Nothing else of the cache is touched.  The page-table entries of
 * the written positions must name existing pages (a precondition, as for the
 * attention entry points).  Returns MLA_ERR_UNSUPPORTED for an unsupported page_size
 * or an unknown kv_dtype, MLA_ERR_INVALID for null pointers (when
 * total_new > 0), batch < 1, total_new < 0, max_pages_per_req < 1 or an
 * int8 or fp8 cache without kv_scale.  total_new == 0 enqueues nothing.
 */
int mla_kv_append(const void* kv_new, const int32_t* cu_seqlens_new, const int32_t* start_pos,
                  void* kv_cache, float* kv_scale, int kv_dtype, const int32_t* page_table,
                  int max_pages_per_req, int batch, int total_new, int page_size, void* hip_stream);

/*
 * Query absorption: q_out[t][h] = [W_UK[h]^T q_nope[t][h] ; q_rope[t][h]], the
 * 576-wide query the attention entry points take [TALK, section
 * "Kernel：让 MLA 真正跑满 GPU": attention over compressed latent rows, query
 * x latent key; the absorbed form is the published MLA formulation: per head
 * the key without position is W_UK[h] c for the latent row c, so
 * q_nope . (W_UK[h] c) = (W_UK[h]^T q_nope) . c].
 *
 *   q        bf16 [tokens, num_heads, 192]: q_nope (128) | q_rope (64)
 *   w_uk_t   bf16 [num_heads, 512, 128]: W_UK[h] transposed (row c holds
 *            W_UK[h][0..127][c]), so that both operands are contiguous in
 *            the contracted index
 *   q_out    bf16 [tokens, num_heads, 576]: 512 absorbed values (fp32
 *            accumulation, rounded to nearest even) then q_rope unchanged
 *
 * Returns MLA_OK (tokens == 0 enqueues nothing), MLA_ERR_INVALID for a null
 * pointer (tokens > 0), tokens < 0 or num_heads < 1, MLA_ERR_UNSUPPORTED when
 * tokens * num_heads * 576 overflows int32, MLA_ERR_HIP.
 */
int mla_q_absorb(const void* q, const void* w_uk_t, void* q_out, int tokens, int num_heads, void* hip_stream);

/*
 * Value up-projection: out[t][h] = W_UV[h] o_lat[t][h], the head output from
 * the 512-wide latent attention output [MLA: the value of a token is W_UV[h] c
 * for its latent row c, and attention weights sum linearly, so the head
 * output is W_UV[h] applied to the weighted mean of latent rows].
 *
 *   o_lat    bf16 [tokens, num_heads, 512] (the attention entry points' out)
 *   w_uv     bf16 [num_heads, 128, 512]: W_UV[h][v][c]
 *   out      bf16 [tokens, num_heads, 128] (fp32 accumulation, rounded to
 *            nearest even)
 *
 * Returns as mla_q_absorb.
 */
int mla_v_up(const void* o_lat, const void* w_uv, void* out, int tokens, int num_heads, void* hip_stream);

/*
 * mla_decode without a workspace argument and without any device allocation,
 * for callers that cannot call hipMalloc: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Arguments, results and
 * errors are those of mla_decode (the same plan and kernels, so the output is
 * bitwise the same), except:
 *
 *   - the split-KV partials live in a scratch array of MLA_NOALLOC_SCRATCH_BYTES
 *     (64 MiB) that the library's code object holds on every GPU it is loaded
 *     on, until the process ends; a shape whose workspace
 *     (mla_splitkv_workspace_size) exceeds it returns MLA_ERR_SCRATCH before
 *     anything is enqueued (with 256 compute units: batch <= 764 at
 *     q_len * num_heads <= 64, batch <= 380 at <= 128);
 *   - every call on one GPU uses that GPU's one array, which keeps the last
 *     call's contents: calls that can overlap on one GPU (other streams, or
 *     other host threads without ordering) race on it and must not be issued.
 *     Calls ordered on one stream are safe (nothing in the array needs to
 *     start at zero: each call writes every byte it reads);
 *   - the first call on a device looks the array's address up (one
 *     hipGetSymbolAddress per device, with that device current), which may
 *     not be done while a stream is being captured: make one call, or the
 *     capture, after a first call outside it.
 */
int mla_decode_noalloc(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                       const int32_t* page_table, int max_pages_per_req, const int32_t* seq_lens,
                       int batch, int q_len, int num_heads, int page_size, int max_seq_len,
                       float softmax_scale, void* out, float* lse, void* hip_stream);

/* Static, human-readable name of a status code. */
const char* mla_status_string(int status);

/*
 * The decode split plan the library would use for these scalars on a device
 * with num_cus compute units (num_cus <= 0: the current device): the number
 * of phase-one workgroups and the workspace bytes.  Exposed for tests and
 * tooling; it is the same pure function mla_decode uses.
 */
int mla_decode_plan(int batch, int num_heads, int q_len, int max_seq_len, int kv_dtype,
                    int num_cus, int* phase1_groups, size_t* workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
