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
#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"
#include "mla_ws.h"

namespace mla {

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

__device__ __forceinline__ WorkTile locate_work(const PrefillArgs& a, int t, int row_blocks);

// The work tile's block: its tokens' rows from the first, the pages its
// last token sees, outputs in place.
__device__ __forceinline__ WsBlock block_of(const PrefillArgs& a, const WorkTile& wt) {
  WsBlock k;
  const size_t row0 = (size_t)(wt.q0 + wt.j0) * a.heads;  // the tile's first query row
  k.q = a.q + row0 * kDqk;
  k.out = a.out + row0 * kDv;
  k.lse = a.lse + row0;
  k.lse_mul = kLn2;
  k.r0 = kBlockRows * wt.rb;
  k.nrows = (wt.j1 - wt.j0) * a.heads;
  k.vis0 = wt.P_b + wt.j0;
  k.heads = a.heads;
  k.b = wt.b;
  k.p_lo = 0;
  k.p_hi = wt.npages;
  k.kv_end = wt.kv_end;
  return k;
}

__device__ __forceinline__ WsArgs ws_args(const PrefillArgs& a) {
  return WsArgs{a.kv, a.kv_scale, a.page_table, a.pt_stride, a.sub, a.scale_log2};
}

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

// bf16 cache: a ring of four stages, two tiles in flight while two are read
// (tile k by the score waves, tile k - 1 by the value waves).  A third stage
// only, with one tile in flight, left the tile's load latency exposed in an
// earlier design (19% slower).
constexpr int kPFStages = 4;

// ---------------------------------------------------------------------------
// Wave-specialised bf16 prefill.  Waves 0-3 compute scores and softmax,
// waves 4-7 the value product (waves w and w + 4 share a SIMD).  The 64
// query rows of a work tile form two 32-row groups rg.  Score wave (rg, kh)
// holds the query fragments of its group's rows (two 16-row MFMA tiles)
// and scores them against rows 16kh .. 16kh+15 of each staged tile, so each
// K fragment read from LDS feeds two MFMAs.  Value wave vq holds the
// accumulators of all 64 rows for value columns 128vq .. 128vq+127, so each
// transposed V fragment read feeds four MFMAs.  Per 32-row tile the waves
// read 74 KB of K and 33 KB of V from LDS; the MFMA work per SIMD is the
// same as with any other split.
//
// Step k (between barriers B1(k) and B2(k), then B2(k) to B1(k+1)):
//  - score waves: take the partner's row max of tile k-1 (written after
//    B2(k-1)), finish the softmax of tile k-1 for their own 16 rows of it
//    (the two partners use the same max, so they make the same rescale
//    decisions), write their half of the probability fragments and the
//    rescale factors, and compute the scores of tile k (the first kKAhead
//    K fragments are requested before the softmax, which covers their
//    latency); after B2(k) they publish tile k's row max;
//  - value waves: at B1(k) issue every load of tile k + 2 (the score waves
//    issue none, so they start on their K reads at once); after B2(k),
//    rescale and run the value product of tile k - 1 from the 16
//    transposed V fragments in registers, re-reading each fragment from
//    tile k's stage as soon as its four MFMAs have taken it.
// The V reads of tile k thus overlap the value MFMAs of tile k - 1 and stay
// out of the score phase: measured, V reads that run into the score waves'
// K reads slow the whole step, so B1 waits for them.
// Each score wave keeps the row sums of its own 16 rows of every tile; the
// two halves are added at the end of the work tile.  Stages k (scores and V
// reads) and k - 1 (V in registers) are in use during step k while k + 1
// and k + 2 load.
// ---------------------------------------------------------------------------

// K prefetch distance (k-steps) of the score waves: the first reads go out
// before the softmax, which covers their latency.  Measured: 4 ahead beat 6
// by 2% and 6 beat 8 (alternating runs on one box).
constexpr int kKAhead = 4;

struct WsLds {
  MLA_LDS uint8_t* ring;
  MLA_LDS float* mx;     // [4 score waves][2 query tiles][64]: row maxes, then row sums
  MLA_LDS uint8_t* pb;   // [2 row groups][2 query tiles][64] x 16 B probability fragments
  MLA_LDS float* al;     // [2 row groups][2 query tiles][64]: rescale factors, then 1 / row sum
  int* pid;              // page ids of the window
};

// One work tile, as a score wave (SCORE) or a value wave.  Both kinds pass
// the same barriers in the same order; each keeps only its own state live.
template <bool SCORE>
__device__ __forceinline__ void ws_work_tile(const WsArgs& a, const WsBlock& k_, const WsLds& L, int w, int lane) {
  const int rg = (w & 3) >> 1;  // score waves: row group
  const int hh = w & 1;         // score waves: tile-row half kh
  const int vq = w & 3;         // value waves: column quarter
  const int g = lane >> 4;
  const int r0 = 32 * rg + (lane & 15);
  const QRow x0 = ws_row(k_, r0), x1 = ws_row(k_, r0 + 16);
  auto stage = [&](int k) { return L.ring + (k % kPFStages) * kStageBytes; };
  MLA_LDS float* const mx_mine = L.mx + 128 * w + lane;
  const MLA_LDS float* const mx_part = L.mx + 128 * (w ^ 1) + lane;
  MLA_LDS uint8_t* const pb_row = L.pb + (128 * rg + lane) * 16;  // query tile j: + 64 * 16 * j
  MLA_LDS float* const al_row = L.al + 128 * rg + lane;           // query tile j: + 64 * j

  // value waves: the byte offsets (within a half page, row t of the half)
  // of this lane's slot in each of the wave's tile loads (load i = lw + 4 j)
  // are the same for every tile; full tiles use them as they are
  constexpr int kMyLoads = (kStageLoads + kLoadWaves - 1) / kLoadWaves;  // 10
  const int lw = __builtin_amdgcn_readfirstlane(w - (kWaves - kLoadWaves));  // wave-uniform
  int ld_off[kMyLoads];
  if (!SCORE) {
#pragma unroll
    for (int j = 0; j < kMyLoads; ++j) ld_off[j] = stage_src(lw + kLoadWaves * j, lane, 0, kTileRows);
  }

  // score-wave state
  bf16x8 q0[kQFrags], q1[kQFrags];
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.f, l1 = 0.f, mx0 = -INFINITY, mx1 = -INFINITY;
  f32x4 sp0 = {0.f, 0.f, 0.f, 0.f}, sp1 = sp0;
  // value-wave state
  f32x4 o[kVQTiles][kVCTiles];
  bf16x4 vb[kVCTiles][2];
  if (SCORE) {
    issue_q(x0.ok ? k_.q + (size_t)x0.qrow * kDqk : nullptr, lane, q0);
    issue_q(x1.ok ? k_.q + (size_t)x1.qrow * kDqk : nullptr, lane, q1);
  } else {
#pragma unroll
    for (int qt = 0; qt < kVQTiles; ++qt)
#pragma unroll
      for (int ct = 0; ct < kVCTiles; ++ct) o[qt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // score waves, step k: softmax of the previous tile, then the scores of tile k (kk < 0: none)
  // (the softmax and the scores are one branch-free block)
  auto score_step = [&](auto with_scores, int kk, int lim0, int lim1) {
    constexpr bool kScores = decltype(with_scores)::value;
    const MLA_LDS uint8_t* kbase = stage(kk < 0 ? 0 : kk) + tile_off(16 * hh + (lane & 15), g);
    bf16x8 kb[kKAhead];
    if constexpr (kScores) {
#pragma unroll
      for (int d = 0; d < kKAhead; ++d) kb[d] = lds_b128(kbase + 64 * d);
    }
    __builtin_amdgcn_sched_barrier(0);  // the first K reads go out before the softmax
    float al0, al1;
    const bf16x4 p0 = softmax_half(sp0, fmaxf(mx0, mx_part[0]), m0, l0, al0);
    const bf16x4 p1 = softmax_half(sp1, fmaxf(mx1, mx_part[64]), m1, l1, al1);
    *reinterpret_cast<MLA_LDS bf16x4*>(pb_row + 8 * hh) = p0;
    *reinterpret_cast<MLA_LDS bf16x4*>(pb_row + 64 * 16 + 8 * hh) = p1;
    al_row[0] = al0;  // the same factors from both partner waves
    al_row[64] = al1;
    if constexpr (kScores) {
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
#pragma unroll
      for (int ks = 0; ks < kQFrags; ++ks) {
        const bf16x8 kf = kb[ks % kKAhead];
        if (ks + kKAhead < kQFrags) kb[ks % kKAhead] = lds_b128(kbase + 64 * (ks + kKAhead));
        if (ks & 1) {
          a1 = mfma16x16x32(kf, q0[ks], a1);
          b1 = mfma16x16x32(kf, q1[ks], b1);
        } else {
          a0 = mfma16x16x32(kf, q0[ks], a0);
          b0 = mfma16x16x32(kf, q1[ks], b0);
        }
      }
      mx0 = mask_half(a0 + a1, hh, lim0, a.scale_log2, lane, sp0);
      mx1 = mask_half(b0 + b1, hh, lim1, a.scale_log2, lane, sp1);
    }
  };
  // value waves: the value product of the tile in vb from the published
  // probabilities; with REFILL, vb is re-read from the stage of tile `next`
  auto value_step = [&](auto refill, int next) {
    value_product<decltype(refill)::value>(L.pb, L.al, vb, o, stage(next), lane, vq);
  };

  for (int plo = k_.p_lo; plo < k_.p_hi; plo += kPWin) {
    const int n = min(kPWin, k_.p_hi - plo);
    lds_barrier();  // the previous window's list and stages are no longer read
    for (int k = threadIdx.x; k < n; k += kWaves * 64)
      L.pid[k] = sub_page(a.page_table, (size_t)k_.b * a.pt_stride, plo + k, a.sub);
    __builtin_amdgcn_s_waitcnt(0);  // the page ids are in LDS (and every earlier load has landed)
    lds_barrier();
    const int ntiles = min(2 * n, (k_.kv_end - kPage * plo + kTileRows - 1) / kTileRows);
    // Only the value waves issue tile loads (kLoadWaves of them), so the
    // score waves start each step on their K reads; the page id of the next
    // tile to issue is read from LDS one step ahead.
    int pid_next = 0;
    auto issue = [&](int k, int pid) {
      const int p = k >> 1;
      const int half = k & 1;
      const int rem = k_.kv_end - kPage * (plo + p);
      const uint8_t* page = a.kv + (size_t)pid * kPageBytes;
      if (rem >= kTileRows * (half + 1)) {  // every row of the tile is the request's
        const uint8_t* hbase = page + (size_t)half * kTileRows * kRowBytes;
#pragma unroll
        for (int j = 0; j < kMyLoads; ++j) {
          const int i = lw + kLoadWaves * j;
          if (i < kStageLoads) lds_dma16(hbase, ld_off[j], stage(k) + i * 1024);
        }
      } else {
        stage_tile<kLoadWaves>(page, half, rem, stage(k), lw, lane);
      }
    };
    auto lim_of = [&](const QRow& x, int k) { return x.ok ? x.vis_last - (kPage * plo + kTileRows * k) : -1; };
    auto wait_for = [&](int k) {  // tile k landed; tile k + 1 may stay in flight
      if (SCORE) return;
      if (k + 1 < ntiles) wait_tile<kLoadWaves>(1, w - (kWaves - kLoadWaves)); else wait_vmcnt<0>();
    };
    if (!SCORE) {
      issue(0, L.pid[0]);
      if (1 < ntiles) issue(1, L.pid[0]);
      pid_next = L.pid[1 < n ? 1 : 0];
    }
    // step 0: scores only
    wait_for(0);
    lds_write_barrier();  // B1(0)
    if (!SCORE && 2 < ntiles) {
      issue(2, pid_next);
      pid_next = L.pid[min(3, 2 * n - 1) >> 1];
    }
    if (SCORE) {
      f32x4 c0, c1;
      scores_2q(stage(0), q0, q1, lane, hh, c0, c1);
      mx0 = mask_half(c0, hh, lim_of(x0, 0), a.scale_log2, lane, sp0);
      mx1 = mask_half(c1, hh, lim_of(x1, 0), a.scale_log2, lane, sp1);
    }
    lds_write_barrier();  // B2(0)
    if (SCORE) {
      mx_mine[0] = mx0;
      mx_mine[64] = mx1;
    } else {
      values_fetch(stage(0), lane, vq, vb);  // V of tile 0
    }
    for (int k = 1; k < ntiles; ++k) {
      wait_for(k);
      lds_write_barrier();  // B1(k)
      if (!SCORE && k + 2 < ntiles) {
        issue(k + 2, pid_next);
        pid_next = L.pid[min(k + 3, 2 * n - 1) >> 1];
      }
      if (SCORE) score_step(std::true_type{}, k, lim_of(x0, k), lim_of(x1, k));
      // B2(k): the probabilities and factors are written; the value waves'
      // V reads of tile k may stay in flight
      if (SCORE)
        lds_write_barrier();
      else
        lds_barrier();
      if (SCORE) {
        mx_mine[0] = mx0;
        mx_mine[64] = mx1;
      } else {
        value_step(std::true_type{}, k);  // tile k - 1, then V of tile k into vb
      }
    }
    // the window's last tile
    lds_write_barrier();  // B1'
    if (SCORE) score_step(std::false_type{}, -1, 0, 0);
    if (SCORE)  // B2'
      lds_write_barrier();
    else
      lds_barrier();
    if (!SCORE) value_step(std::false_type{}, 0);
  }

  // row totals: each score wave holds the sums of its own tile rows
  lds_write_barrier();  // the last value product is done with the probabilities and factors
  float s0 = 0.f, s1 = 0.f;
  if (SCORE) {
    wait_vmcnt<0>();  // query loads of a tile that saw no cache rows
    s0 = wave_sum_rows(l0);
    s1 = wave_sum_rows(l1);
    mx_mine[0] = s0;
    mx_mine[64] = s1;
  }
  lds_write_barrier();
  if (SCORE) {
    const float t0 = s0 + mx_part[0], t1 = s1 + mx_part[64];  // the same sums in both partners
    if (hh == 0) {
      al_row[0] = t0 > 0.f ? 1.0f / t0 : 0.f;
      al_row[64] = t1 > 0.f ? 1.0f / t1 : 0.f;
      if (g == 0) {
        if (x0.ok) k_.lse[x0.qrow] = t0 > 0.f ? (m0 + fast_log2(t0)) * k_.lse_mul : -INFINITY;
        if (x1.ok) k_.lse[x1.qrow] = t1 > 0.f ? (m1 + fast_log2(t1)) * k_.lse_mul : -INFINITY;
      }
    }
  }
  lds_write_barrier();
  if (!SCORE) ws_store_rows(k_, L.al, o, lane, vq);
}

__global__ __launch_bounds__(kWaves * 64, 2) void prefill_persistent_ws(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring_raw[kPFStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) float mx_raw[4 * 2 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t pb_raw[2 * 2 * 64 * 16];
  __shared__ __attribute__((aligned(16))) float al_raw[2 * 2 * 64];
  __shared__ int s_pid[kPWin];
  __shared__ int s_tile;
  const WsLds L{(MLA_LDS uint8_t*)ring_raw, (MLA_LDS float*)mx_raw, (MLA_LDS uint8_t*)pb_raw,
                (MLA_LDS float*)al_raw, s_pid};
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int total_tiles = a.tile_cum[a.batch];
  const int block_rows = a.tok_per_tile * a.heads;
  const int row_blocks = (block_rows + kBlockRows - 1) / kBlockRows;
  for (;;) {
    __syncthreads();  // previous tile fully done (stages, page list, s_tile)
    if (threadIdx.x == 0) s_tile = atomicAdd(a.counter, 1);
    __syncthreads();
    const int t = s_tile;
    if (t >= total_tiles) break;
    const WsBlock k = block_of(a, locate_work(a, t, row_blocks));
    if (w < 4)
      ws_work_tile<true>(ws_args(a), k, L, w, lane);
    else
      ws_work_tile<false>(ws_args(a), k, L, w, lane);
  }
}

template <int CODE>
__global__ __launch_bounds__(kWaves * 64, 2) void prefill_persistent_ws_codes(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t cvt_raw[3 * kStageBytes];
  __shared__ __attribute__((aligned(16))) float tsc_raw[3 * kTileRows];
  __shared__ __attribute__((aligned(16))) float mx_raw[4 * 2 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t pb_raw[2 * 2 * 64 * 16];
  __shared__ __attribute__((aligned(16))) float al_raw[2 * 2 * 64];
  __shared__ int s_pid[kPWin];
  __shared__ int s_tile;
  const WsCodesLds L{(MLA_LDS uint8_t*)cvt_raw, (MLA_LDS float*)tsc_raw, (MLA_LDS float*)mx_raw,
                     (MLA_LDS uint8_t*)pb_raw, (MLA_LDS float*)al_raw, s_pid};
  const int lane = threadIdx.x & 63;
  const int w = wave_uniform(threadIdx.x >> 6);
  const int total_tiles = a.tile_cum[a.batch];
  const int block_rows = a.tok_per_tile * a.heads;
  const int row_blocks = (block_rows + kBlockRows - 1) / kBlockRows;
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) s_tile = atomicAdd(a.counter, 1);
    __syncthreads();
    const int t = s_tile;
    if (t >= total_tiles) break;
    const WsBlock k = wave_uniform(block_of(a, locate_work(a, t, row_blocks)));
    if (w < 4)
      ws_codes_range<true, CODE>(ws_args(a), k, L, w, lane);
    else
      ws_codes_range<false, CODE>(ws_args(a), k, L, w, lane);
  }
}

hipError_t launch_prefill(const PrefillPlan& plan, const PrefillArgs& args, int kv_dtype, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_worklist, dim3(1), dim3(256), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kv_dtype == 1)
    hipLaunchKernelGGL(prefill_persistent_ws_codes<kCodeInt8>, dim3(plan.grid), dim3(kWaves * 64), 0, stream, args);
  else if (kv_dtype == 2)
    hipLaunchKernelGGL(prefill_persistent_ws_codes<kCodeFp8>, dim3(plan.grid), dim3(kWaves * 64), 0, stream, args);
  else
    hipLaunchKernelGGL(prefill_persistent_ws, dim3(plan.grid), dim3(kWaves * 64), 0, stream, args);
  return hipGetLastError();
}

}  // namespace mla
