// C ABI of the MLA library: argument checks, split planning, workspace
// layout and launches.  See include/mla.h for the contract of each call.
//
// Planning follows [TALK "构建面向 Agentic 推理的下一代 LLM 推理引擎", section
// "Kernel：让 MLA 真正跑满 GPU"]: the split parameters and the workspace size
// are computed at run time from the shape and cached.  Here the plan is a
// pure function of (shape scalars, compute-unit count); the cache memoises
// it per (device, shape) and is guarded by a mutex.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <map>
#include <mutex>
#include <tuple>

#include "mla.h"
#include "mla_internal.h"

namespace mla {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

DecodePlan plan_decode(int batch, int heads, int q_len, int max_seq_len, int kv_dtype, int num_cus) {
  (void)kv_dtype;
  DecodePlan p{};
  const int rows = q_len * heads;
  p.waves = 8;
  // One phase-one workgroup per compute unit (the ring of staged tiles takes
  // most of a CU's LDS), and at least one page of work per workgroup: on
  // short caches the call is latency-bound, and more, shorter shares plus
  // the merge measured faster than fewer, longer ones (256 rows: 12.3 us
  // with 4 workgroups against 15.9 with 1; 4 x 2K rows: 14.2 against 22.2).
  //
  // A block of more than 64 folded rows runs as two row blocks (blockIdx.y), each a
  // workgroup streaming the same share: the grid then has one workgroup per CU in all,
  // so that every workgroup is resident at once, and with the share count a multiple
  // of 8 the two readers of a share land on the same XCD (workgroups are dealt to the
  // XCDs round-robin by linear index), where the second read of each page hits its L2.
  const long long pages_max = (long long)batch * ceil_div(max_seq_len, kPage);
  const int row_blocks = (rows + kBlockRowsHost - 1) / kBlockRowsHost;
  long long g = num_cus > 0 ? num_cus / row_blocks : 1;
  const long long cap = pages_max;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  p.grid = (int)g;
  if (p.grid > 1) {
    const size_t slots = (size_t)(p.grid + batch) * rows;
    size_t off = 0;
    p.part_o_off = off;
    off = align256(off + slots * kDv * sizeof(uint16_t));  // bf16 partial outputs
    p.part_lse_off = off;
    off = align256(off + slots * sizeof(float));
    p.cum_off = off;
    off = align256(off + (size_t)(batch + 1) * sizeof(int32_t));
    p.workspace_bytes = off;
  }
  return p;
}

PrefillPlan plan_prefill(int batch, int heads, int max_q_len, int total_q, int max_seq_len,
                         int kv_dtype, int num_cus) {
  (void)max_q_len;
  (void)total_q;
  (void)max_seq_len;
  (void)kv_dtype;
  PrefillPlan p{};
  // A work tile is as many whole query tokens as fit in one block of 64
  // query rows; a token with more than 64 heads is one tile per 64-row block.
  p.tok_per_tile = heads >= 64 ? 1 : 64 / heads;
  p.waves = 8;
  p.grid = num_cus > 0 ? num_cus : 1;
  size_t off = 0;
  p.counter_off = off;
  off = align256(off + sizeof(int32_t));
  p.order_off = off;
  off = align256(off + (size_t)batch * sizeof(int32_t));
  p.tile_cum_off = off;
  off = align256(off + (size_t)(batch + 1) * sizeof(int32_t));
  p.workspace_bytes = off;
  return p;
}

}  // namespace mla

using namespace mla;

namespace {

std::mutex g_mu;
constexpr int kMaxDevs = 64;
int g_cus[kMaxDevs] = {};  // device -> compute units (0: not yet asked)
std::map<std::tuple<int, int, int, int, int, int>, DecodePlan> g_decode_plans;

// Compute units of the current device (MLA_NUM_CUS overrides, for planning
// without a GPU).  Returns MLA_OK or MLA_ERR_HIP.
int device_cus(int* dev_out, int* cus_out) {
  if (const char* env = std::getenv("MLA_NUM_CUS")) {
    const int v = std::atoi(env);
    if (v > 0) {
      *dev_out = -1;
      *cus_out = v;
      return MLA_OK;
    }
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevs) return MLA_ERR_HIP;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cus[dev] > 0) {
      *dev_out = dev;
      *cus_out = g_cus[dev];
      return MLA_OK;
    }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  g_cus[dev] = cus;
  *dev_out = dev;
  *cus_out = cus;
  return MLA_OK;
}

int cached_decode_plan(int batch, int heads, int q_len, int max_seq_len, int kv_dtype, DecodePlan* out) {
  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != MLA_OK) return rc;
  const auto key = std::make_tuple(dev * 100000 + cus, batch, heads, q_len, max_seq_len, kv_dtype);
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_decode_plans.find(key);
  if (it == g_decode_plans.end()) {
    if (g_decode_plans.size() > 4096) g_decode_plans.clear();
    it = g_decode_plans.emplace(key, plan_decode(batch, heads, q_len, max_seq_len, kv_dtype, cus)).first;
  }
  *out = it->second;
  return MLA_OK;
}

// Shapes a decode call (uniform or per-request query counts) can take.
bool decode_shape(int batch, int num_heads, int max_q_len, int total_q) {
  return (long long)max_q_len * num_heads <= MLA_MAX_DECODE_ROWS &&
         (long long)batch * max_q_len >= total_q;
}

// Page sizes: whole numbers of 64-row sub-pages (the kernels' unit), up to
// MLA_MAX_PAGE_SIZE rows.
bool known_page_size(int page_size) {
  return page_size >= MLA_PAGE_SIZE && page_size <= MLA_MAX_PAGE_SIZE && page_size % MLA_PAGE_SIZE == 0;
}

bool known_dtype(int kv_dtype) {
  return kv_dtype == MLA_KV_BF16 || kv_dtype == MLA_KV_INT8 || kv_dtype == MLA_KV_FP8;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime or launch error";
    case MLA_ERR_SCRATCH: return "split-KV workspace larger than the fixed scratch of mla_decode_noalloc";
    default: return "unknown status";
  }
}

int mla_decode_plan(int batch, int num_heads, int q_len, int max_seq_len, int kv_dtype, int num_cus,
                    int* phase1_groups, size_t* workspace_bytes) {
  if (!phase1_groups || !workspace_bytes) return MLA_ERR_INVALID;
  if (batch < 1 || num_heads < 1 || q_len < 1 || max_seq_len < q_len) return MLA_ERR_INVALID;
  if (!known_dtype(kv_dtype)) return MLA_ERR_UNSUPPORTED;
  if ((long long)q_len * num_heads > MLA_MAX_DECODE_ROWS) return MLA_ERR_UNSUPPORTED;
  DecodePlan p{};
  if (num_cus > 0) {
    p = plan_decode(batch, num_heads, q_len, max_seq_len, kv_dtype, num_cus);
  } else {
    const int rc = cached_decode_plan(batch, num_heads, q_len, max_seq_len, kv_dtype, &p);
    if (rc != MLA_OK) return rc;
  }
  *phase1_groups = p.grid;
  *workspace_bytes = p.workspace_bytes;
  return MLA_OK;
}

int mla_splitkv_workspace_size(int batch, int num_heads, int max_q_len, int total_q, int max_seq_len,
                               int kv_dtype, size_t* bytes_out) {
  if (!bytes_out) return MLA_ERR_INVALID;
  *bytes_out = 0;
  if (batch < 1 || num_heads < 1 || max_q_len < 0 || total_q < 0 || max_seq_len < 1) return MLA_ERR_INVALID;
  if (!known_dtype(kv_dtype)) return MLA_ERR_UNSUPPORTED;
  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != MLA_OK) return rc;
  size_t bytes = 0;
  if (max_q_len >= 1 && max_seq_len >= max_q_len && decode_shape(batch, num_heads, max_q_len, total_q)) {
    DecodePlan d{};
    const int rc2 = cached_decode_plan(batch, num_heads, max_q_len, max_seq_len, kv_dtype, &d);
    if (rc2 != MLA_OK) return rc2;
    bytes = d.workspace_bytes;
  }
  if (num_heads <= MLA_MAX_HEADS) {
    const PrefillPlan pp = plan_prefill(batch, num_heads, max_q_len, total_q, max_seq_len, kv_dtype, cus);
    if (pp.workspace_bytes > bytes) bytes = pp.workspace_bytes;
  }
  *bytes_out = bytes;
  return MLA_OK;
}

}  // extern "C"

namespace {

// Decode with uniform (cu_q null: q_len tokens per request) or per-request
// query counts (cu_q: device offsets, q_len the largest count, total_q the
// total).  Host-scalar checks come first, before any HIP call.  With
// `fixed_scratch`, the workspace arguments are ignored: the plan is computed
// without the plan cache and the split-KV scratch is the library's fixed device
// array (MLA_ERR_SCRATCH when the plan needs more).
int decode_impl(const void* q, const int32_t* cu_q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                const int32_t* page_table, int max_pages_per_req, const int32_t* seq_lens, int batch,
                int total_q, int q_len, int num_heads, int page_size, int max_seq_len, float softmax_scale,
                void* out, float* lse, void* workspace, size_t workspace_bytes, void* hip_stream,
                bool fixed_scratch = false) {
  if (batch < 1 || q_len < 1 || num_heads < 1 || max_pages_per_req < 1 || max_seq_len < 1)
    return MLA_ERR_INVALID;
  if (total_q < 0 || (long long)total_q > (long long)batch * q_len) return MLA_ERR_INVALID;
  // with no query token nothing is read or written: only the scalars are checked
  if (total_q > 0 && (!q || !kv_cache || !page_table || !seq_lens || !out || !lse)) return MLA_ERR_INVALID;
  if (!known_dtype(kv_dtype)) return MLA_ERR_UNSUPPORTED;
  if (kv_dtype != MLA_KV_BF16 && !kv_scale) return MLA_ERR_INVALID;
  if (!known_page_size(page_size)) return MLA_ERR_UNSUPPORTED;
  if ((long long)q_len * num_heads > MLA_MAX_DECODE_ROWS) return MLA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID;
  if (max_seq_len < q_len) return MLA_ERR_INVALID;
  if ((long long)max_pages_per_req * page_size < max_seq_len) return MLA_ERR_INVALID;
  if ((long long)max_pages_per_req * page_size > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if ((long long)batch * max_pages_per_req > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if ((long long)batch * q_len * num_heads > 0x7fffffffLL / MLA_DIM_QK) return MLA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return MLA_ERR_INVALID;

  if (total_q == 0) return MLA_OK;  // no query rows: nothing to compute or write

  DecodePlan plan{};
  if (fixed_scratch) {
    int dev = 0, cus = 0;
    const int rc = device_cus(&dev, &cus);
    if (rc != MLA_OK) return rc;
    plan = plan_decode(batch, num_heads, q_len, max_seq_len, kv_dtype, cus);
    if (plan.workspace_bytes > kNoAllocScratchBytes) return MLA_ERR_SCRATCH;
    workspace = nullptr;
    if (plan.workspace_bytes > 0 && noalloc_scratch(&workspace) != hipSuccess) return MLA_ERR_HIP;
    workspace_bytes = kNoAllocScratchBytes;
  } else {
    const int rc = cached_decode_plan(batch, num_heads, q_len, max_seq_len, kv_dtype, &plan);
    if (rc != MLA_OK) return rc;
    if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
      return MLA_ERR_WORKSPACE;
  }

  DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv_cache);
  a.kv_scale = kv_scale;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.cu_q = cu_q;
  a.pt_stride = max_pages_per_req;
  a.sub = page_size / MLA_PAGE_SIZE;
  a.max_pages = max_pages_per_req * a.sub;
  a.batch = batch;
  a.q_len = q_len;
  a.heads = num_heads;
  a.rows = q_len * num_heads;
  a.grid = plan.grid;
  // the bf16 decode's first tile is requested before the lengths arrive, on the
  // guess that every request holds max_seq_len rows (uniform query counts only)
  a.guess_pages = cu_q ? 0 : (max_seq_len + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE;
  a.scale_log2 = softmax_scale * kLog2e;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  if (plan.grid > 1) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.part_o = reinterpret_cast<uint16_t*>(ws + plan.part_o_off);
    a.part_lse = reinterpret_cast<float*>(ws + plan.part_lse_off);
    a.cum_pages = reinterpret_cast<int32_t*>(ws + plan.cum_off);
  }
  const hipError_t e = launch_decode(plan, a, kv_dtype, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

int mla_decode(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
               const int32_t* page_table, int max_pages_per_req, const int32_t* seq_lens, int batch,
               int q_len, int num_heads, int page_size, int max_seq_len, float softmax_scale, void* out,
               float* lse, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (batch < 1 || q_len < 1) return MLA_ERR_INVALID;
  return decode_impl(q, nullptr, kv_cache, kv_scale, kv_dtype, page_table, max_pages_per_req, seq_lens, batch,
                     (int)std::min<long long>((long long)batch * q_len, 0x7fffffffLL), q_len, num_heads,
                     page_size, max_seq_len, softmax_scale, out, lse, workspace, workspace_bytes, hip_stream);
}

int mla_decode_noalloc(const void* q, const void* kv_cache, const float* kv_scale, int kv_dtype,
                       const int32_t* page_table, int max_pages_per_req, const int32_t* seq_lens, int batch,
                       int q_len, int num_heads, int page_size, int max_seq_len, float softmax_scale, void* out,
                       float* lse, void* hip_stream) {
  if (batch < 1 || q_len < 1) return MLA_ERR_INVALID;
  return decode_impl(q, nullptr, kv_cache, kv_scale, kv_dtype, page_table, max_pages_per_req, seq_lens, batch,
                     (int)std::min<long long>((long long)batch * q_len, 0x7fffffffLL), q_len, num_heads,
                     page_size, max_seq_len, softmax_scale, out, lse, nullptr, 0, hip_stream, true);
}

int mla_decode_varlen(const void* q, const int32_t* cu_seqlens_q, const void* kv_cache, const float* kv_scale,
                      int kv_dtype, const int32_t* page_table, int max_pages_per_req, const int32_t* seq_lens,
                      int batch, int total_q, int max_q_len, int num_heads, int page_size, int max_seq_len,
                      float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  if (!cu_seqlens_q) return MLA_ERR_INVALID;
  return decode_impl(q, cu_seqlens_q, kv_cache, kv_scale, kv_dtype, page_table, max_pages_per_req, seq_lens,
                     batch, total_q, max_q_len, num_heads, page_size, max_seq_len, softmax_scale, out, lse,
                     workspace, workspace_bytes, hip_stream);
}

int mla_prefill_varlen(const void* q, const int32_t* cu_seqlens_q, const int32_t* prefix_lens,
                       const void* kv_cache, const float* kv_scale, int kv_dtype,
                       const int32_t* page_table, int max_pages_per_req, int batch, int total_q,
                       int max_q_len, int max_seq_len, int num_heads, int page_size, float softmax_scale,
                       void* out, float* lse, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!q || !cu_seqlens_q || !prefix_lens || !kv_cache || !page_table || !out || !lse)
    return MLA_ERR_INVALID;
  if (batch < 1 || num_heads < 1 || max_pages_per_req < 1 || total_q < 0 || max_q_len < 0 ||
      max_seq_len < 1)
    return MLA_ERR_INVALID;
  if (total_q < max_q_len || max_seq_len < max_q_len) return MLA_ERR_INVALID;
  if (!known_dtype(kv_dtype)) return MLA_ERR_UNSUPPORTED;
  if (kv_dtype != MLA_KV_BF16 && !kv_scale) return MLA_ERR_INVALID;
  if (!known_page_size(page_size)) return MLA_ERR_UNSUPPORTED;
  if (num_heads > MLA_MAX_HEADS) return MLA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID;
  if ((long long)max_pages_per_req * page_size < max_seq_len) return MLA_ERR_INVALID;
  if ((long long)max_pages_per_req * page_size > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if ((long long)batch * max_pages_per_req > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if ((long long)total_q * num_heads > 0x7fffffffLL / MLA_DIM_QK) return MLA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return MLA_ERR_INVALID;
  if (total_q == 0) return MLA_OK;

  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != MLA_OK) return rc;
  const PrefillPlan plan = plan_prefill(batch, num_heads, max_q_len, total_q, max_seq_len, kv_dtype, cus);
  if (!workspace || workspace_bytes < plan.workspace_bytes) return MLA_ERR_WORKSPACE;

  PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.cu_seqlens = cu_seqlens_q;
  a.prefix_lens = prefix_lens;
  a.kv = static_cast<const uint8_t*>(kv_cache);
  a.kv_scale = kv_scale;
  a.page_table = page_table;
  a.pt_stride = max_pages_per_req;
  a.sub = page_size / MLA_PAGE_SIZE;
  a.max_pages = max_pages_per_req * a.sub;
  a.batch = batch;
  a.total_q = total_q;
  a.heads = num_heads;
  a.tok_per_tile = plan.tok_per_tile;
  a.grid = plan.grid;
  a.scale_log2 = softmax_scale * kLog2e;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.counter = reinterpret_cast<int32_t*>(ws + plan.counter_off);
  a.order = reinterpret_cast<int32_t*>(ws + plan.order_off);
  a.tile_cum = reinterpret_cast<int32_t*>(ws + plan.tile_cum_off);
  const hipError_t e = launch_prefill(plan, a, kv_dtype, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_kv_append(const void* kv_new, const int32_t* cu_seqlens_new, const int32_t* start_pos,
                  void* kv_cache, float* kv_scale, int kv_dtype, const int32_t* page_table,
                  int max_pages_per_req, int batch, int total_new, int page_size, void* hip_stream) {
  if (batch < 1 || total_new < 0 || max_pages_per_req < 1) return MLA_ERR_INVALID;
  if (!known_dtype(kv_dtype)) return MLA_ERR_UNSUPPORTED;
  if (!known_page_size(page_size)) return MLA_ERR_UNSUPPORTED;
  if (total_new > 0 && (!kv_new || !cu_seqlens_new || !start_pos || !kv_cache || !page_table))
    return MLA_ERR_INVALID;
  if (kv_dtype != MLA_KV_BF16 && !kv_scale) return MLA_ERR_INVALID;
  if ((long long)batch * max_pages_per_req > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if ((long long)max_pages_per_req * page_size > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if (total_new == 0) return MLA_OK;

  AppendArgs a{};
  a.kv_new = static_cast<const uint16_t*>(kv_new);
  a.cu = cu_seqlens_new;
  a.start_pos = start_pos;
  a.kv = static_cast<uint8_t*>(kv_cache);
  a.kv_scale = kv_dtype != MLA_KV_BF16 ? kv_scale : nullptr;  // the kernel keys on it
  a.code = kv_dtype;
  a.page_table = page_table;
  a.pt_stride = max_pages_per_req;
  a.sub = page_size / MLA_PAGE_SIZE;
  a.max_pages = max_pages_per_req * a.sub;
  a.batch = batch;
  a.total_new = total_new;
  const hipError_t e = launch_append(a, kv_dtype, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_q_absorb(const void* q, const void* w_uk_t, void* q_out, int tokens, int num_heads, void* hip_stream) {
  if (tokens < 0 || num_heads < 1) return MLA_ERR_INVALID;
  if (tokens == 0) return MLA_OK;
  if (!q || !w_uk_t || !q_out) return MLA_ERR_INVALID;
  if ((long long)tokens * num_heads > 0x7fffffffLL / MLA_DIM_QK) return MLA_ERR_UNSUPPORTED;
  const size_t dq = MLA_DIM_NOPE + MLA_DIM_ROPE;
  GemmArgs g{};
  g.a = static_cast<const uint16_t*>(q);
  g.a_row = (size_t)num_heads * dq;
  g.a_head = dq;
  g.bt = static_cast<const uint16_t*>(w_uk_t);
  g.b_row = MLA_DIM_NOPE;
  g.b_head = (size_t)MLA_DIM_V * MLA_DIM_NOPE;
  g.c = static_cast<uint16_t*>(q_out);
  g.c_row = (size_t)num_heads * MLA_DIM_QK;
  g.c_head = MLA_DIM_QK;
  g.m = tokens;
  g.n = MLA_DIM_V;
  g.k = MLA_DIM_NOPE;
  g.rope_src = g.a + MLA_DIM_NOPE;
  g.rope_src_row = g.a_row;
  g.rope_src_head = g.a_head;
  g.rope_dst = g.c + MLA_DIM_V;
  g.rope_dst_row = g.c_row;
  g.rope_dst_head = g.c_head;
  g.rope_cols = MLA_DIM_ROPE;
  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != MLA_OK) return rc;
  const hipError_t e = launch_gemm(g, num_heads, cus, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_v_up(const void* o_lat, const void* w_uv, void* out, int tokens, int num_heads, void* hip_stream) {
  if (tokens < 0 || num_heads < 1) return MLA_ERR_INVALID;
  if (tokens == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_INVALID;
  if ((long long)tokens * num_heads > 0x7fffffffLL / MLA_DIM_QK) return MLA_ERR_UNSUPPORTED;
  GemmArgs g{};
  g.a = static_cast<const uint16_t*>(o_lat);
  g.a_row = (size_t)num_heads * MLA_DIM_V;
  g.a_head = MLA_DIM_V;
  g.bt = static_cast<const uint16_t*>(w_uv);
  g.b_row = MLA_DIM_V;
  g.b_head = (size_t)MLA_DIM_VHEAD * MLA_DIM_V;
  g.c = static_cast<uint16_t*>(out);
  g.c_row = (size_t)num_heads * MLA_DIM_VHEAD;
  g.c_head = MLA_DIM_VHEAD;
  g.m = tokens;
  g.n = MLA_DIM_VHEAD;
  g.k = MLA_DIM_V;
  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != MLA_OK) return rc;
  const hipError_t e = launch_gemm(g, num_heads, cus, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
