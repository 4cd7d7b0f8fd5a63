// Host-side structures shared between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kDqk = 576;                      // row width: 512 latent + 64 rope
constexpr int kDv = 512;                       // value width
constexpr int kPage = 64;                      // rows per page (= one LDS tile)
constexpr int kBlockRowsHost = 64;             // folded query rows per decode workgroup
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Arguments of the decode kernels (passed by value as kernel arguments).
struct DecodeArgs {
  const uint16_t* q;          // bf16 [batch * q_len, heads, 576]
  const uint8_t* kv;          // pages, bf16 or int8 rows
  const float* kv_scale;      // int8 only
  const int32_t* page_table;  // [batch, max_pages]
  const int32_t* seq_lens;    // [batch]
  const int32_t* cu_q;        // [batch + 1] first query token of each request, or null: b * q_len
  int max_pages;              // 64-row sub-pages a request can hold (page-table entries * sub)
  int pt_stride;              // page-table entries per request
  int sub;                    // 64-row sub-pages per page (page size / 64)
  int batch;
  int q_len;                  // query tokens per request (with cu_q: the largest)
  int heads;
  int rows;                   // q_len * heads: folded query rows of one request (with cu_q: at most)
  int grid;                   // phase-one workgroups
  int guess_pages;            // 64-row sub-pages of a request of max_seq_len rows (0: no guessed start)
  float scale_log2;           // softmax_scale * log2(e)
  uint16_t* out;              // bf16 [batch * rows, 512]
  float* lse;                 // fp32 [batch * rows]
  uint16_t* part_o;           // workspace: bf16 [(grid + batch) * rows, 512], normalised partial outputs
  float* part_lse;            // workspace: [(grid + batch) * rows], log2 units
  int32_t* cum_pages;         // workspace: [batch + 1] page prefix sums
};

// Arguments of the prefill kernels.
struct PrefillArgs {
  const uint16_t* q;          // bf16 [total_q, heads, 576]
  const int32_t* cu_seqlens;  // [batch + 1]
  const int32_t* prefix_lens; // [batch]
  const uint8_t* kv;
  const float* kv_scale;
  const int32_t* page_table;
  int max_pages;              // 64-row sub-pages a request can hold (page-table entries * sub)
  int pt_stride;              // page-table entries per request
  int sub;                    // 64-row sub-pages per page (page size / 64)
  int batch;
  int total_q;
  int heads;
  int tok_per_tile;           // query tokens per work tile (tile rows = tok_per_tile * heads)
  int grid;
  float scale_log2;
  uint16_t* out;
  float* lse;
  int32_t* order;             // workspace: [batch] requests, most expensive first
  int32_t* tile_cum;          // workspace: [batch + 1] cumulative tiles in that order
  int32_t* counter;           // workspace: work-queue head
};

struct AppendArgs {
  const uint16_t* kv_new;     // bf16 [total_new, 576]
  const int32_t* cu;          // [batch + 1] new-row offsets
  const int32_t* start_pos;   // [batch] logical position of each request's first new row
  uint8_t* kv;                // pages, bf16 or int8 rows, written in place
  float* kv_scale;            // int8 only: [num_pages, 64]
  const int32_t* page_table;  // [batch, pt_stride]
  int max_pages;              // 64-row sub-pages a request can hold (page-table entries * sub)
  int pt_stride;              // page-table entries per request
  int sub;                    // 64-row sub-pages per page (page size / 64)
  int batch;
  int total_new;
  int code;                   // scaled caches: 1 INT8, 2 FP8 (E4M3)
};

// One NT product per head: C[m][n] = sum_k A[m][k] Bt[n][k]; element strides.
// With rope_cols > 0, the workgroups of the first column tile also copy
// rope_cols values per row from rope_src to rope_dst.
struct GemmArgs {
  const uint16_t* a;
  size_t a_row, a_head;
  const uint16_t* bt;
  size_t b_row, b_head;
  uint16_t* c;
  size_t c_row, c_head;
  int m, n, k;                // (n, k): (512, 128) or (128, 512)
  const uint16_t* rope_src;
  size_t rope_src_row, rope_src_head;
  uint16_t* rope_dst;
  size_t rope_dst_row, rope_dst_head;
  int rope_cols;              // a multiple of 8, or 0
};

struct DecodePlan {
  int grid;                   // phase-one workgroups (1: single pass, no merge)
  int waves;                  // waves per workgroup (4 or 8)
  size_t part_o_off, part_lse_off, cum_off;
  size_t workspace_bytes;
};

struct PrefillPlan {
  int grid;
  int waves;
  int tok_per_tile;
  size_t order_off, tile_cum_off, counter_off;
  size_t workspace_bytes;
};

DecodePlan plan_decode(int batch, int heads, int q_len, int max_seq_len, int kv_dtype, int num_cus);
PrefillPlan plan_prefill(int batch, int heads, int max_q_len, int total_q, int max_seq_len,
                         int kv_dtype, int num_cus);

hipError_t launch_decode(const DecodePlan& plan, const DecodeArgs& args, int kv_dtype, hipStream_t stream);

// The fixed split-KV scratch of mla_decode_noalloc: a device array of this many bytes
// in the library's code object, one per GPU.  Returns its address on the current device
// (looked up once per device, with that device current).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_prefill(const PrefillPlan& plan, const PrefillArgs& args, int kv_dtype, hipStream_t stream);
hipError_t launch_append(const AppendArgs& args, int kv_dtype, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& g, int heads, int cus, hipStream_t stream);

}  // namespace mla
