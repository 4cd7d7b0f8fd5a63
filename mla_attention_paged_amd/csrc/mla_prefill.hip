// Variable-length MLA prefill over a paged latent cache, persistent grid.
//
// Sources (web pages on the TokenSpeed inference engine):
//   [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎", AICon 2026 talk
//          transcript.  Section "Kernel：让 MLA 真正跑满 GPU": agent requests
//          hit a cached prefix and append a few hundred tokens, so Q and KV
//          lengths differ per request and the kernel batches them with no
//          padding.  Section "跨平台 Kernel 设计": on MI355X a persistent
//          prefill kernel balances the scheduling across compute units.
//
// Work decomposition.  A work tile is up to `tok_per_tile` consecutive new
// tokens of one request and one block of at most 64 of their query rows
// (tok_per_tile * heads <= 64, or one token whose heads fill two blocks).  Its cost is proportional to the cached rows its last token sees
// (prefix + position + 1).  A one-workgroup kernel orders the requests by the
// cost of their most expensive tile, most expensive first, and lays out the
// cumulative tile counts in that order; the tiles of a request are handed out
// last-token-first.  A persistent grid of one workgroup per compute unit then
// takes tiles from an atomic counter until the list is exhausted: the long
// tiles start first and the short ones fill the tail (longest processing
// time first).  Every tile streams its request's pages 0 .. through the same
// LDS pipeline as decode; only the pages that hold a row some query token of
// the tile can see are read, and only the diagonal pages are masked.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kPWin = 128;  // page ids staged per window

__device__ __forceinline__ int p_clamp(int L, int max_pages) {
  L = L < 0 ? 0 : L;
  const int cap = max_pages * kPage;
  return L > cap ? cap : L;
}

// One workgroup: order requests by tile cost, lay out cumulative tile
// counts, reset the queue head.
__global__ __launch_bounds__(256) void prefill_worklist(PrefillArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // rank sort by cost (descending), ties by request index
  for (int b = tid; b < a.batch; b += 256) {
    const int n = a.cu_seqlens[b + 1] - a.cu_seqlens[b];
    const long long cb = n > 0 ? (long long)a.prefix_lens[b] + n : -1;
    int rank = 0;
    for (int o = 0; o < a.batch; ++o) {
      const int no = a.cu_seqlens[o + 1] - a.cu_seqlens[o];
      const long long co = no > 0 ? (long long)a.prefix_lens[o] + no : -1;
      rank += (co > cb) || (co == cb && o < b);
    }
    a.order[rank] = b;
  }
  if (tid == 0) *a.counter = 0;
  __syncthreads();
  if (tid < 64) {
    int run = 0;
    for (int base = 0; base < a.batch; base += 64) {
      const int k = base + lane;
      int nt = 0;
      if (k < a.batch) {
        const int b = a.order[k];
        const int n = a.cu_seqlens[b + 1] - a.cu_seqlens[b];
        const int row_blocks = (a.tok_per_tile * a.heads + 63) / 64;
        nt = n > 0 ? (n + a.tok_per_tile - 1) / a.tok_per_tile * row_blocks : 0;
      }
      int incl = nt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
      }
      if (k < a.batch) a.tile_cum[k] = run + incl - nt;
      run += __shfl(incl, 63);
    }
    if (lane == 0) a.tile_cum[a.batch] = run;
  }
}

// A work tile, located from its queue index: the request, its new-token
// range, and the cache rows its last token sees.
struct WorkTile {
  int b, q0, j0, j1, P_b, kv_end, npages, rb;
};

__device__ __forceinline__ WorkTile locate_work(const PrefillArgs& a, int t, int row_blocks) {
  // order position k with tile_cum[k] <= t < tile_cum[k+1]
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.tile_cum[mid] <= t) lo = mid; else hi = mid - 1;
  }
  WorkTile w;
  w.b = a.order[lo];
  w.q0 = a.cu_seqlens[w.b];
  const int n_b = a.cu_seqlens[w.b + 1] - w.q0;
  const int ntok = (n_b + a.tok_per_tile - 1) / a.tok_per_tile;
  const int local = t - a.tile_cum[lo];
  const int jt = ntok - 1 - local / row_blocks;        // last token tiles first
  w.rb = local - (local / row_blocks) * row_blocks;    // row block
  w.j0 = jt * a.tok_per_tile;                          // first new token of the tile
  w.j1 = min(n_b, w.j0 + a.tok_per_tile);              // one past its last
  w.P_b = a.prefix_lens[w.b];
  const int L_b = p_clamp(w.P_b + n_b, a.max_pages);
  w.kv_end = min(L_b, w.P_b + w.j1);                   // rows the tile's last token sees
  w.npages = w.kv_end > 0 ? (w.kv_end + kPage - 1) / kPage : 0;
  return w;
}

// Rows of a work tile owned by a wave of 16 rows: row r of the tile is head
// r % heads of token j0 + r / heads.
struct WaveRows {
  bool wave_rows, row_ok;
  int qrow;      // index of the lane's query row in [total_q * heads]
  int vis_last;  // last cache row its token sees
};

__device__ __forceinline__ WaveRows wave_rows_of(const PrefillArgs& a, const WorkTile& wt, int w, int lane,
                                                 int block_rows) {
  WaveRows x;
  const int r = kBlockRows * wt.rb + 16 * (w & 3) + (lane & 15);
  x.wave_rows = kBlockRows * wt.rb + 16 * (w & 3) < block_rows;
  const int tok_in_tile = r / a.heads;
  const int head = r - tok_in_tile * a.heads;
  const int j = wt.j0 + tok_in_tile;                   // this lane's new-token index
  x.row_ok = x.wave_rows && r < block_rows && j < wt.j1;
  x.qrow = (wt.q0 + j) * a.heads + head;
  x.vis_last = wt.P_b + j;                             // last visible cache row of this query token
  return x;
}

__device__ __forceinline__ void store_rows(const PrefillArgs& a, const RowState& st, const WaveRows& x, int half,
                                           int lane) {
  float inv, lse2;
  finish_row(st, inv, lse2);
  if (x.row_ok) {
    const int g = lane >> 4;
    uint16_t* dst = a.out + (size_t)x.qrow * kDv + (kDv / 2) * half + 4 * g;
#pragma unroll
    for (int ct = 0; ct < kOHalf; ++ct) {
      const f32x4 v = st.o[ct] * inv;
      bf16x4 h;
      h[0] = (__bf16)v[0]; h[1] = (__bf16)v[1]; h[2] = (__bf16)v[2]; h[3] = (__bf16)v[3];
      *reinterpret_cast<bf16x4*>(dst + 16 * ct) = h;
    }
    if (g == 0 && half == 0) a.lse[x.qrow] = lse2 * kLn2;
  }
}

// INT8 or FP8 cache (CODE): the lockstep core.  Every tile is converted to
// bf16 in LDS by all waves after its barrier, then scored, normalised and
// accumulated before the next tile starts; R::stages - 1 tiles are in flight.
template <int CODE>
__global__ __launch_bounds__(kWaves * 64, 2) void prefill_persistent_codes(PrefillArgs a) {
  using R = Ring<true>;
  __shared__ __attribute__((aligned(1024))) uint8_t ring_raw[R::stages * R::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t cvt_raw[kStageBytes];
  __shared__ __attribute__((aligned(16))) f32x4 xchg_raw[kWaves * 64];
  MLA_LDS uint8_t* const ring = (MLA_LDS uint8_t*)ring_raw;
  MLA_LDS uint8_t* const cvt = (MLA_LDS uint8_t*)cvt_raw;
  MLA_LDS f32x4* const xchg = (MLA_LDS f32x4*)xchg_raw;
  __shared__ int s_pid[kPWin];
  __shared__ int s_tile;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int half = w >> 2;
  const int total_tiles = a.tile_cum[a.batch];
  const int block_rows = a.tok_per_tile * a.heads;                 // query rows of a token tile
  const int row_blocks = (block_rows + kBlockRows - 1) / kBlockRows;
  MLA_LDS f32x4* const xmine = xchg + 64 * w + lane;
  const MLA_LDS f32x4* const xpart = xchg + 64 * (w ^ 4) + lane;

  RowState st;
  bf16x8 qf[kQFrags];

  for (;;) {
    __syncthreads();  // previous tile fully done (stages, page list, s_tile)
    if (threadIdx.x == 0) s_tile = atomicAdd(a.counter, 1);
    __syncthreads();
    const int t = s_tile;
    if (t >= total_tiles) break;
    const WorkTile wt = locate_work(a, t, row_blocks);
    const WaveRows x = wave_rows_of(a, wt, w, lane, block_rows);
    if (x.wave_rows) {
      load_q(x.row_ok ? a.q + (size_t)x.qrow * kDqk : nullptr, lane, qf);
      reset_state(st);
    }

    for (int plo = 0; plo < wt.npages; plo += kPWin) {
      const int n = min(kPWin, wt.npages - plo);
      __syncthreads();
      for (int k = threadIdx.x; k < n; k += kWaves * 64)
        s_pid[k] = sub_page(a.page_table, (size_t)wt.b * a.pt_stride, plo + k, a.sub);
      __syncthreads();
      // tiles of 32 rows: only those holding a row the tile's last token sees
      const int ntiles = min(2 * n, (wt.kv_end - kPage * plo + kTileRows - 1) / kTileRows);
      auto issue = [&](int k) {
        const int p = k >> 1;
        MLA_LDS uint8_t* stage = ring + (k % R::stages) * R::stage_bytes;
        const int rem = wt.kv_end - kPage * (plo + p);
        stage_tile_i8<kWaves>(a.kv + (size_t)s_pid[p] * kI8PageBytes, a.kv_scale + (size_t)s_pid[p] * kPage,
                              k & 1, rem, stage, w, lane);
      };
      const int pre = min(R::stages - 1, ntiles);
      for (int k = 0; k < pre; ++k) issue(k);
      for (int k = 0; k < ntiles; ++k) {
        const int t0 = kPage * plo + kTileRows * k;  // first cache row of tile k
        wait_tile<kWaves, R::loads>(min(R::stages - 2, ntiles - 1 - k), w);
        lds_barrier();
        if (k + R::stages - 1 < ntiles) issue(k + R::stages - 1);
        const MLA_LDS uint8_t* stage = ring + (k % R::stages) * R::stage_bytes;
        convert_code_tile<CODE>(stage, cvt, threadIdx.x);
        lds_write_barrier();
        if (x.wave_rows) {
          const int lim = x.row_ok ? x.vis_last - t0 : -1;
          attend_tile<true>(cvt, qf, lim, a.scale_log2, lane, half, xmine, xpart, st,
                            reinterpret_cast<const MLA_LDS float*>(stage + kI8CodeBytes));
        } else {
          lds_write_barrier();  // the exchange barrier inside attend_tile
        }
      }
    }
    if (x.wave_rows) store_rows(a, st, x, half, lane);
  }
}

// bf16 cache: the pipelined core over a ring of four stages, two tiles in
// flight.  Step k of a window waits for tile k, passes a barrier, starts
// tile k + 2, and computes the scores of tile k while the softmax and value
// product of tile k - 1 run in the same basic block.  The partner waves swap
// score halves through one slot per wave: the slot of tile k - 1 is read
// right after the first barrier, and a second barrier at the end of the
// step orders those reads before the slot is overwritten with tile k.  (The
// double-buffered slot of the decode kernel would not fit beside a fourth
// stage in 160 KB of LDS; a third stage only, with one tile in flight,
// leaves the tile's load latency exposed: measured 19% slower.)
constexpr int kPFStages = 4;

__global__ __launch_bounds__(kWaves * 64, 2) void prefill_persistent_bf16(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring_raw[kPFStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) f32x4 xchg_raw[kWaves * 64];
  MLA_LDS uint8_t* const ring = (MLA_LDS uint8_t*)ring_raw;
  MLA_LDS f32x4* const xchg = (MLA_LDS f32x4*)xchg_raw;
  __shared__ int s_pid[kPWin];
  __shared__ int s_tile;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int half = w >> 2;
  const int total_tiles = a.tile_cum[a.batch];
  const int block_rows = a.tok_per_tile * a.heads;
  const int row_blocks = (block_rows + kBlockRows - 1) / kBlockRows;
  MLA_LDS f32x4* const xmine = xchg + 64 * w + lane;
  const MLA_LDS f32x4* const xpart = xchg + 64 * (w ^ 4) + lane;
  auto stage = [&](int k) { return ring + (k % kPFStages) * kStageBytes; };

  RowState st;
  bf16x8 qf[kQFrags];

  for (;;) {
    __syncthreads();  // previous tile fully done (stages, page list, s_tile)
    if (threadIdx.x == 0) s_tile = atomicAdd(a.counter, 1);
    __syncthreads();
    const int t = s_tile;
    if (t >= total_tiles) break;
    const WorkTile wt = locate_work(a, t, row_blocks);
    const WaveRows x = wave_rows_of(a, wt, w, lane, block_rows);
    if (x.wave_rows) {
      issue_q(x.row_ok ? a.q + (size_t)x.qrow * kDqk : nullptr, lane, qf);
      reset_state(st);
    }

    for (int plo = 0; plo < wt.npages; plo += kPWin) {
      const int n = min(kPWin, wt.npages - plo);
      __syncthreads();  // the previous window's list and stages are no longer read
      for (int k = threadIdx.x; k < n; k += kWaves * 64)
        s_pid[k] = sub_page(a.page_table, (size_t)wt.b * a.pt_stride, plo + k, a.sub);
      __syncthreads();
      const int ntiles = min(2 * n, (wt.kv_end - kPage * plo + kTileRows - 1) / kTileRows);
      auto issue = [&](int k) {
        const int p = k >> 1;
        stage_tile<kWaves>(a.kv + (size_t)s_pid[p] * kPageBytes, k & 1, wt.kv_end - kPage * (plo + p), stage(k),
                           w, lane);
      };
      auto lim_of = [&](int k) { return x.row_ok ? x.vis_last - (kPage * plo + kTileRows * k) : -1; };
      auto wait_for = [&](int k) {  // tile k landed; tile k + 1 may stay in flight
        if (k + 1 < ntiles) wait_tile<kWaves>(1, w); else wait_vmcnt<0>();
      };
      issue(0);
      if (1 < ntiles) issue(1);
      // first step: scores only (its wait also covers the query loads)
      wait_for(0);
      lds_write_barrier();
      if (2 < ntiles) issue(2);
      f32x4 s_prev = {0.f, 0.f, 0.f, 0.f};
      if (x.wave_rows) s_prev = tile_scores(stage(0), qf, lane, half);
      int prev_lim = lim_of(0);
      for (int k = 1; k < ntiles; ++k) {
        if (x.wave_rows) *xmine = s_prev;  // scores of tile k - 1
        wait_for(k);
        lds_write_barrier();
        if (k + 2 < ntiles) issue(k + 2);
        if (x.wave_rows) {
          const f32x4 other = *xpart;
          const f32x4 lo = half == 0 ? s_prev : other;
          const f32x4 hi = half == 0 ? other : s_prev;
          s_prev = tile_step(stage(k), stage(k - 1), qf, lo, hi, prev_lim, a.scale_log2, lane, half, st);
        }
        prev_lim = lim_of(k);
        lds_write_barrier();  // every wave has read its partner's slot of tile k - 1
      }
      // last tile of the window
      if (x.wave_rows) *xmine = s_prev;
      lds_write_barrier();
      if (x.wave_rows) {
        const f32x4 other = *xpart;
        const f32x4 lo = half == 0 ? s_prev : other;
        const f32x4 hi = half == 0 ? other : s_prev;
        float alpha;
        const bf16x8 pb = tile_softmax(lo, hi, prev_lim, a.scale_log2, lane, st, alpha);
        rescale_o(st, alpha);
        tile_values(stage(ntiles - 1), pb, lane, half, st);
      }
    }
    if (x.wave_rows) {
      wait_vmcnt<0>();  // query loads of a tile that saw no cache rows
      store_rows(a, st, x, half, lane);
    }
  }
}

hipError_t launch_prefill(const PrefillPlan& plan, const PrefillArgs& args, int kv_dtype, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_worklist, dim3(1), dim3(256), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kv_dtype == 1)
    hipLaunchKernelGGL(prefill_persistent_codes<kCodeInt8>, dim3(plan.grid), dim3(kWaves * 64), 0, stream, args);
  else if (kv_dtype == 2)
    hipLaunchKernelGGL(prefill_persistent_codes<kCodeFp8>, dim3(plan.grid), dim3(kWaves * 64), 0, stream, args);
  else
    hipLaunchKernelGGL(prefill_persistent_bf16, dim3(plan.grid), dim3(kWaves * 64), 0, stream, args);
  return hipGetLastError();
}

}  // namespace mla
