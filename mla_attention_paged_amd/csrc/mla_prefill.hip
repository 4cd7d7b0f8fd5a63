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

namespace mla {

constexpr int kPWin = 256;  // page ids staged per window (a pipeline restart per window)

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

// Scores of this wave's 16 tile rows against two 16-row query tiles: each K
// fragment is read once and used by both tiles' MFMAs (four accumulator
// chains).  s_j[e]: tile row 16kh + 4(lane>>4) + e, query row lane & 15 of
// query tile j.
__device__ __forceinline__ void scores_2q(const MLA_LDS uint8_t* tile, const bf16x8 (&q0)[kQFrags],
                                          const bf16x8 (&q1)[kQFrags], int lane, int kh, f32x4& s0, f32x4& s1) {
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const MLA_LDS uint8_t* kbase = tile + tile_off(16 * kh + r16, g);
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
  bf16x8 kb[kKDepth + 1];
#pragma unroll
  for (int d = 0; d < kKDepth; ++d) kb[d] = lds_b128(kbase + 64 * d);
#pragma unroll
  for (int ks = 0; ks < kQFrags; ++ks) {
    if (ks + kKDepth < kQFrags) kb[(ks + kKDepth) % (kKDepth + 1)] = lds_b128(kbase + 64 * (ks + kKDepth));
    const bf16x8 kf = kb[ks % (kKDepth + 1)];
    if (ks & 1) {
      a1 = mfma16x16x32(kf, q0[ks], a1);
      b1 = mfma16x16x32(kf, q1[ks], b1);
    } else {
      a0 = mfma16x16x32(kf, q0[ks], a0);
      b0 = mfma16x16x32(kf, q1[ks], b0);
    }
  }
  s0 = a0 + a1;
  s1 = b0 + b1;
}

// Scale to log2 units and mask (tile row tt visible when tt <= lim); returns
// the row max over the wave's 16 tile rows (equal on the row's four lanes).
__device__ __forceinline__ float mask_half(f32x4 acc, int kh, int lim, float scale_log2, int lane, f32x4& s) {
  const int g = lane >> 4;
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = 16 * kh + 4 * g + e <= lim ? acc[e] * scale_log2 : -INFINITY;
    s[e] = v;
    mx = fmaxf(mx, v);
  }
  return wave_max_rows(mx);
}

// Online softmax of this wave's 16 rows of a tile, given the row max over
// all 32 (mx): raises the running max m past the slack, returns the four
// probabilities (bf16, the wave's half of the value product's B operand)
// and the factor alpha for the accumulators; lh is this lane's share of the
// row sum over the wave's rows of every tile.
__device__ __forceinline__ bf16x4 softmax_half(const f32x4& s, float mx, float& m, float& lh, float& alpha) {
  const float m_new = mx > m + kRescaleSlack ? mx : m;
  alpha = m_new == m ? 1.f : fast_exp2(m - m_new);
  m = m_new;
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  bf16x4 p;
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = fast_exp2(s[e] - m_use);
    ps += v;
    p[e] = (__bf16)v;
  }
  lh = lh * alpha + ps;
  return p;
}

// The value waves: value wave vq owns value columns 128 vq .. 128 vq + 127
// (eight 16-column tiles) of all four 16-row query tiles of the 64-row block,
// so each transposed V fragment read from LDS feeds four MFMAs (a split by
// 32-row groups and column halves fed two: twice the V bytes read per flop).
constexpr int kVQTiles = 4;   // 16-row query tiles per value wave
constexpr int kVCTiles = 8;   // 16-column value tiles per value wave

// Lane's transposed-read address of column tile 0 of quarter vq in a staged tile.
__device__ __forceinline__ const MLA_LDS uint8_t* vq_base(const MLA_LDS uint8_t* tile, int lane, int vq) {
  const int g = lane >> 4;
  const int i16 = lane & 15;
  return tile + (4 * g + (i16 >> 2)) * kLdsPitch + 4 * (i16 & 3) * 2 + 256 * vq;
}

// All eight V fragments of the wave's quarter of a tile (32 registers).
__device__ __forceinline__ void values_fetch(const MLA_LDS uint8_t* tile, int lane, int vq,
                                             bf16x4 (&vb)[kVCTiles][2]) {
  const MLA_LDS uint8_t* vbase = vq_base(tile, lane, vq);
#pragma unroll
  for (int ct = 0; ct < kVCTiles; ++ct) {
    vb[ct][0] = lds_tr16(vbase + 32 * ct);
    vb[ct][1] = lds_tr16(vbase + 16 * kLdsPitch + 32 * ct);
  }
}

// The value product of the tile in vb for the four query tiles.  With REFILL,
// each column tile's two V fragments are re-read from `next` (the following
// tile's stage) as soon as its four MFMAs have taken them, so the next tile's
// V reads overlap this tile's value MFMAs.
template <bool REFILL>
__device__ __forceinline__ void values_mfma(bf16x4 (&vb)[kVCTiles][2], const bf16x8 (&p)[kVQTiles],
                                            f32x4 (&o)[kVQTiles][kVCTiles], const MLA_LDS uint8_t* next, int lane,
                                            int vq) {
  const MLA_LDS uint8_t* vbase = nullptr;
  if constexpr (REFILL) vbase = vq_base(next, lane, vq);
#pragma unroll
  for (int ct = 0; ct < kVCTiles; ++ct) {
    const bf16x4 v0 = vb[ct][0], v1 = vb[ct][1];
    bf16x8 va;
    va[0] = v0[0]; va[1] = v0[1]; va[2] = v0[2]; va[3] = v0[3];
    va[4] = v1[0]; va[5] = v1[1]; va[6] = v1[2]; va[7] = v1[3];
#pragma unroll
    for (int qt = 0; qt < kVQTiles; ++qt) o[qt][ct] = mfma16x16x32(va, p[qt], o[qt][ct]);
    if constexpr (REFILL) {
      vb[ct][0] = lds_tr16(vbase + 32 * ct);
      vb[ct][1] = lds_tr16(vbase + 16 * kLdsPitch + 32 * ct);
    }
  }
}

// Value waves, after B2: the published probabilities and rescale factors of
// the four query tiles (query tile qt = 2 row group + tile of the group:
// entry 64 qt + lane), the rescale when some row's max was raised, then the
// product.
template <bool REFILL>
__device__ __forceinline__ void value_product(const MLA_LDS uint8_t* pb, const MLA_LDS float* al,
                                              bf16x4 (&vb)[kVCTiles][2], f32x4 (&o)[kVQTiles][kVCTiles],
                                              const MLA_LDS uint8_t* next, int lane, int vq) {
  bf16x8 p[kVQTiles];
  float f[kVQTiles];
#pragma unroll
  for (int qt = 0; qt < kVQTiles; ++qt) {
    p[qt] = *reinterpret_cast<const MLA_LDS bf16x8*>(pb + (64 * qt + lane) * 16);
    f[qt] = al[64 * qt + lane];
  }
  if (__ballot(f[0] != 1.f || f[1] != 1.f || f[2] != 1.f || f[3] != 1.f)) {
#pragma unroll
    for (int qt = 0; qt < kVQTiles; ++qt)
#pragma unroll
      for (int ct = 0; ct < kVCTiles; ++ct) o[qt][ct] *= f[qt];
  }
  values_mfma<REFILL>(vb, p, o, next, lane, vq);
}

// Value waves, at the end of a work tile: normalise (al holds 1 / row sum) and
// store the wave's 128 columns of each of the block's rows.
__device__ __forceinline__ void store_rows(const PrefillArgs& a, const WorkTile& wt, const MLA_LDS float* al,
                                           const f32x4 (&o)[kVQTiles][kVCTiles], int lane, int vq, int block_rows);

// K prefetch distance (k-steps) of the score waves: the first reads go out
// before the softmax, which covers their latency.  Measured: 4 ahead beat 6
// by 2% and 6 beat 8 (alternating runs on one box).
constexpr int kKAhead = 4;

// Waves that issue the bf16 tile loads (the value waves, the last four).
constexpr int kLoadWaves = 4;

// A query row of a work tile: row r of the tile is head r % heads of token
// j0 + r / heads.
struct QRow {
  bool ok;       // the row exists
  int qrow;      // its index in [total_q * heads]
  int vis_last;  // last cache row its token sees
};

__device__ __forceinline__ QRow qrow_of(const PrefillArgs& a, const WorkTile& wt, int r, int block_rows) {
  QRow x;
  const int tok = r / a.heads;
  const int head = r - tok * a.heads;
  const int j = wt.j0 + tok;
  x.ok = r < block_rows && j < wt.j1;
  x.qrow = (wt.q0 + j) * a.heads + head;
  x.vis_last = wt.P_b + j;
  return x;
}

__device__ __forceinline__ void store_rows(const PrefillArgs& a, const WorkTile& wt, const MLA_LDS float* al,
                                           const f32x4 (&o)[kVQTiles][kVCTiles], int lane, int vq, int block_rows) {
  const int col = 128 * vq + 4 * (lane >> 4);
#pragma unroll
  for (int qt = 0; qt < kVQTiles; ++qt) {
    const QRow x = qrow_of(a, wt, kBlockRows * wt.rb + 16 * qt + (lane & 15), block_rows);
    const float inv = al[64 * qt + lane];
    if (x.ok) {
      uint16_t* dst = a.out + (size_t)x.qrow * kDv + col;
#pragma unroll
      for (int ct = 0; ct < kVCTiles; ++ct) {
        const f32x4 v = o[qt][ct] * inv;
        bf16x4 h;
        h[0] = (__bf16)v[0]; h[1] = (__bf16)v[1]; h[2] = (__bf16)v[2]; h[3] = (__bf16)v[3];
        *reinterpret_cast<bf16x4*>(dst + 16 * ct) = h;
      }
    }
  }
}

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
__device__ __forceinline__ void ws_work_tile(const PrefillArgs& a, const WorkTile& wt, const WsLds& L, int w,
                                             int lane, int block_rows) {
  const int rg = (w & 3) >> 1;  // score waves: row group
  const int hh = w & 1;         // score waves: tile-row half kh
  const int vq = w & 3;         // value waves: column quarter
  const int g = lane >> 4;
  const int r0 = kBlockRows * wt.rb + 32 * rg + (lane & 15);
  const QRow x0 = qrow_of(a, wt, r0, block_rows), x1 = qrow_of(a, wt, r0 + 16, block_rows);
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
    issue_q(x0.ok ? a.q + (size_t)x0.qrow * kDqk : nullptr, lane, q0);
    issue_q(x1.ok ? a.q + (size_t)x1.qrow * kDqk : nullptr, lane, q1);
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

  for (int plo = 0; plo < wt.npages; plo += kPWin) {
    const int n = min(kPWin, wt.npages - plo);
    lds_barrier();  // the previous window's list and stages are no longer read
    for (int k = threadIdx.x; k < n; k += kWaves * 64)
      L.pid[k] = sub_page(a.page_table, (size_t)wt.b * a.pt_stride, plo + k, a.sub);
    __builtin_amdgcn_s_waitcnt(0);  // the page ids are in LDS (and every earlier load has landed)
    lds_barrier();
    const int ntiles = min(2 * n, (wt.kv_end - kPage * plo + kTileRows - 1) / kTileRows);
    // Only the value waves issue tile loads (kLoadWaves of them), so the
    // score waves start each step on their K reads; the page id of the next
    // tile to issue is read from LDS one step ahead.
    int pid_next = 0;
    auto issue = [&](int k, int pid) {
      const int p = k >> 1;
      const int half = k & 1;
      const int rem = wt.kv_end - kPage * (plo + p);
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
        if (x0.ok) a.lse[x0.qrow] = t0 > 0.f ? (m0 + fast_log2(t0)) * kLn2 : -INFINITY;
        if (x1.ok) a.lse[x1.qrow] = t1 > 0.f ? (m1 + fast_log2(t1)) * kLn2 : -INFINITY;
      }
    }
  }
  lds_write_barrier();
  if (!SCORE) store_rows(a, wt, L.al, o, lane, vq, block_rows);
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
    const WorkTile wt = locate_work(a, t, row_blocks);
    if (w < 4)
      ws_work_tile<true>(a, wt, L, w, lane, block_rows);
    else
      ws_work_tile<false>(a, wt, L, w, lane, block_rows);
  }
}

// ---------------------------------------------------------------------------
// INT8 / FP8 cache (CODE) on the wave-specialised core (K prefetch depth
// kKAheadC: the score waves here also hold the row scales).  The value waves
// bring each tile's codes straight into registers with ordinary global loads
// (value thread i: row i / 8 of the tile, 72 consecutive code bytes; thread
// i < 32 also row i's scale), a step ahead, and widen them to exact bf16
// into one of three converted tiles in LDS (the tile's 32 row scales beside
// it) in the value phase, next to their value MFMAs.  No code bytes pass
// through LDS and no wave issues loads in the score phase.  Step k:
//  - B1(k): tile k is converted (in step k - 1);
//  - score waves: softmax of tile k - 1 (probabilities times their row's
//    scale, selected to 0 on masked rows so that a non-finite scale there
//    cannot leak; the row sums take the unscaled probabilities), then the
//    scores of tile k from its converted tile, each row's score times its
//    scale; value waves: the V fragments of tile k - 1;
//  - B2(k): the probabilities of tile k - 1 are published;
//  - value waves: the value product of tile k - 1, the conversion of tile
//    k + 1 (its codes were requested in step k - 1) and the loads of tile
//    k + 2's codes into the registers that just freed up.
// ---------------------------------------------------------------------------

// mask_half with each tile row's scale (sc: rows 16kh + 4(lane>>4) + e).
__device__ __forceinline__ float mask_half_sc(f32x4 acc, f32x4 sc, int kh, int lim, float scale_log2, int lane,
                                              f32x4& s) {
  const int g = lane >> 4;
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = 16 * kh + 4 * g + e <= lim ? acc[e] * scale_log2 * sc[e] : -INFINITY;
    s[e] = v;
    mx = fmaxf(mx, v);
  }
  return wave_max_rows(mx);
}

// softmax_half whose published probabilities carry their row's scale.
__device__ __forceinline__ bf16x4 softmax_half_sc(const f32x4& s, f32x4 sc, float mx, float& m, float& lh,
                                                  float& alpha) {
  const float m_new = mx > m + kRescaleSlack ? mx : m;
  alpha = m_new == m ? 1.f : fast_exp2(m - m_new);
  m = m_new;
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  bf16x4 p;
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = fast_exp2(s[e] - m_use);
    ps += v;
    p[e] = (__bf16)(s[e] == -INFINITY ? 0.f : v * sc[e]);
  }
  lh = lh * alpha + ps;
  return p;
}

constexpr int kKAheadC = 3;

// One tile's codes in a value thread's registers (see above).
constexpr int kCodeUnits = kI8RowBytes / 8 / 8;  // 9 units of 8 codes

struct CodeRegs {
  u32x2 c[kCodeUnits];
  float sc;  // value threads 0 .. 31: row scale of tile row `thread`
};

// Request tile `half` (rows 32 half ..) of a page: rows at or past `rem` re-read
// row 0's codes; their scales are read as they are and never used unmasked.
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ page, const float* __restrict__ spage,
                                           int half, int rem, int vt, CodeRegs& r) {
  const int t = vt >> 3;
  const int row = kTileRows * half + t;
  const uint8_t* src = page + (size_t)(row < rem ? row : 0) * kI8RowBytes + 8 * kCodeUnits * (vt & 7);
#pragma unroll
  for (int i = 0; i < kCodeUnits; ++i) r.c[i] = *reinterpret_cast<const u32x2*>(src + 8 * i);
  r.sc = vt < kTileRows ? spage[kTileRows * half + vt] : 0.f;
}

// Widen a tile's codes into a converted tile (pitch 1184, like a staged bf16
// tile) and its scales into `tsc`.
template <int CODE>
__device__ __forceinline__ void store_codes(const CodeRegs& r, MLA_LDS uint8_t* cvt, MLA_LDS float* tsc, int vt) {
  MLA_LDS uint8_t* dst = cvt + (vt >> 3) * kLdsPitch + 16 * kCodeUnits * (vt & 7);
#pragma unroll
  for (int i = 0; i < kCodeUnits; ++i) {
    u32x4 o;
    o[0] = codepair_to_bf16<CODE, 0>(r.c[i][0]); o[1] = codepair_to_bf16<CODE, 1>(r.c[i][0]);
    o[2] = codepair_to_bf16<CODE, 0>(r.c[i][1]); o[3] = codepair_to_bf16<CODE, 1>(r.c[i][1]);
    *reinterpret_cast<MLA_LDS u32x4*>(dst + 16 * i) = o;
  }
  if (vt < kTileRows) tsc[vt] = r.sc;
}

struct WsCodesLds {
  MLA_LDS uint8_t* cvt;  // three converted tiles (bf16, pitch 1184)
  MLA_LDS float* tsc;    // their row scales, 32 each
  MLA_LDS float* mx;
  MLA_LDS uint8_t* pb;
  MLA_LDS float* al;
  int* pid;
};

template <bool SCORE, int CODE>
__device__ __forceinline__ void ws_codes_work_tile(const PrefillArgs& a, const WorkTile& wt, const WsCodesLds& L,
                                                   int w, int lane, int block_rows) {
  const int rg = (w & 3) >> 1;  // score waves: row group
  const int hh = w & 1;         // score waves: tile-row half kh
  const int vq = w & 3;         // value waves: column quarter
  const int vt = threadIdx.x - (kWaves - kLoadWaves) * 64;  // value waves: thread 0 .. 255
  const int g = lane >> 4;
  const int r0 = kBlockRows * wt.rb + 32 * rg + (lane & 15);
  const QRow x0 = qrow_of(a, wt, r0, block_rows), x1 = qrow_of(a, wt, r0 + 16, block_rows);
  auto cvt_of = [&](int k) { return L.cvt + (k % 3) * kStageBytes; };
  auto tsc_of = [&](int k) { return L.tsc + (k % 3) * kTileRows; };
  auto tsc4 = [&](int k) {  // this lane's four row scales of tile k (score waves: rows 16kh + 4g + e)
    return *reinterpret_cast<const MLA_LDS f32x4*>(tsc_of(k) + 16 * hh + 4 * g);
  };
  MLA_LDS float* const mx_mine = L.mx + 128 * w + lane;
  const MLA_LDS float* const mx_part = L.mx + 128 * (w ^ 1) + lane;
  MLA_LDS uint8_t* const pb_row = L.pb + (128 * rg + lane) * 16;
  MLA_LDS float* const al_row = L.al + 128 * rg + lane;

  bf16x8 q0[kQFrags], q1[kQFrags];
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.f, l1 = 0.f, mx0 = -INFINITY, mx1 = -INFINITY;
  f32x4 sp0 = {0.f, 0.f, 0.f, 0.f}, sp1 = sp0;
  f32x4 o[kVQTiles][kVCTiles];
  bf16x4 vb[kVCTiles][2];
  CodeRegs rc;  // value waves: the codes of the next tile to convert
  if (SCORE) {
    issue_q(x0.ok ? a.q + (size_t)x0.qrow * kDqk : nullptr, lane, q0);
    issue_q(x1.ok ? a.q + (size_t)x1.qrow * kDqk : nullptr, lane, q1);
  } else {
#pragma unroll
    for (int qt = 0; qt < kVQTiles; ++qt)
#pragma unroll
      for (int ct = 0; ct < kVCTiles; ++ct) o[qt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto score_tile = [&](int kk, int lim0, int lim1) {
    f32x4 c0, c1;
    scores_2q(cvt_of(kk), q0, q1, lane, hh, c0, c1);
    const f32x4 sc = tsc4(kk);
    mx0 = mask_half_sc(c0, sc, hh, lim0, a.scale_log2, lane, sp0);
    mx1 = mask_half_sc(c1, sc, hh, lim1, a.scale_log2, lane, sp1);
  };
  // score waves, step kk: softmax of tile kprev, then (with_scores) the scores of tile kk
  auto score_step = [&](auto with_scores, int kk, int kprev, int lim0, int lim1) {
    constexpr bool kScores = decltype(with_scores)::value;
    const MLA_LDS uint8_t* kbase = cvt_of(kk < 0 ? 0 : kk) + tile_off(16 * hh + (lane & 15), g);
    bf16x8 kb[kKAheadC];
    if constexpr (kScores) {
#pragma unroll
      for (int d = 0; d < kKAheadC; ++d) kb[d] = lds_b128(kbase + 64 * d);
    }
    __builtin_amdgcn_sched_barrier(0);  // the first K reads go out before the softmax
    const f32x4 scp = tsc4(kprev);
    float al0, al1;
    const bf16x4 p0 = softmax_half_sc(sp0, scp, fmaxf(mx0, mx_part[0]), m0, l0, al0);
    const bf16x4 p1 = softmax_half_sc(sp1, scp, fmaxf(mx1, mx_part[64]), m1, l1, al1);
    *reinterpret_cast<MLA_LDS bf16x4*>(pb_row + 8 * hh) = p0;
    *reinterpret_cast<MLA_LDS bf16x4*>(pb_row + 64 * 16 + 8 * hh) = p1;
    al_row[0] = al0;
    al_row[64] = al1;
    if constexpr (kScores) {
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
#pragma unroll
      for (int ks = 0; ks < kQFrags; ++ks) {
        const bf16x8 kf = kb[ks % kKAheadC];
        if (ks + kKAheadC < kQFrags) kb[ks % kKAheadC] = lds_b128(kbase + 64 * (ks + kKAheadC));
        if (ks & 1) {
          a1 = mfma16x16x32(kf, q0[ks], a1);
          b1 = mfma16x16x32(kf, q1[ks], b1);
        } else {
          a0 = mfma16x16x32(kf, q0[ks], a0);
          b0 = mfma16x16x32(kf, q1[ks], b0);
        }
      }
      const f32x4 sc = tsc4(kk);
      mx0 = mask_half_sc(a0 + a1, sc, hh, lim0, a.scale_log2, lane, sp0);
      mx1 = mask_half_sc(b0 + b1, sc, hh, lim1, a.scale_log2, lane, sp1);
    }
  };

  for (int plo = 0; plo < wt.npages; plo += kPWin) {
    const int n = min(kPWin, wt.npages - plo);
    lds_barrier();  // the previous window's page ids and converted tiles are no longer read
    for (int k = threadIdx.x; k < n; k += kWaves * 64)
      L.pid[k] = sub_page(a.page_table, (size_t)wt.b * a.pt_stride, plo + k, a.sub);
    __builtin_amdgcn_s_waitcnt(0);  // the page ids are in LDS
    lds_barrier();
    const int ntiles = min(2 * n, (wt.kv_end - kPage * plo + kTileRows - 1) / kTileRows);
    auto lim_of = [&](const QRow& x, int k) { return x.ok ? x.vis_last - (kPage * plo + kTileRows * k) : -1; };
    // tile k's codes (tiles past the window's last re-read the last one, so
    // that the register sets always hold defined data; they are converted into
    // a buffer nobody reads)
    auto load = [&](int k, CodeRegs& r) {
      if constexpr (!SCORE) {
        const int kk = min(k, ntiles - 1);
        const int p = kk >> 1;
        const int pid = L.pid[p];
        load_codes(a.kv + (size_t)pid * kI8PageBytes, a.kv_scale + (size_t)pid * kPage, kk & 1,
                   wt.kv_end - kPage * (plo + p), vt, r);
      }
    };
    auto convert = [&](int k, const CodeRegs& r) {
      if constexpr (!SCORE) store_codes<CODE>(r, cvt_of(k), tsc_of(k), vt);
    };
    auto value_step = [&](auto refill, int next) {
      value_product<decltype(refill)::value>(L.pb, L.al, vb, o, cvt_of(next), lane, vq);
    };
    // steps k >= 1; `rn` holds the codes of tile k + 1
    auto step = [&](int k, CodeRegs& rn) {
      lds_write_barrier();  // B1(k): tile k converted
      if (SCORE) {
        score_step(std::true_type{}, k, k - 1, lim_of(x0, k), lim_of(x1, k));
      } else {
        convert(k + 1, rn);
        load(k + 2, rn);
      }
      lds_write_barrier();  // B2(k): the probabilities of tile k - 1 are published
      if (SCORE) {
        mx_mine[0] = mx0;
        mx_mine[64] = mx1;
      } else {
        value_step(std::true_type{}, k);  // tile k - 1, then V of tile k into vb
      }
    };

    load(0, rc);
    convert(0, rc);
    load(1, rc);
    lds_write_barrier();  // B1(0): tile 0 converted
    if (SCORE) score_tile(0, lim_of(x0, 0), lim_of(x1, 0));
    lds_write_barrier();  // B2(0)
    if (SCORE) {
      mx_mine[0] = mx0;
      mx_mine[64] = mx1;
    } else {
      convert(1, rc);
      load(2, rc);
      values_fetch(cvt_of(0), lane, vq, vb);  // V of tile 0
    }
    for (int k = 1; k < ntiles; ++k) step(k, rc);
    lds_write_barrier();  // B1'
    if (SCORE) score_step(std::false_type{}, -1, ntiles - 1, 0, 0);
    lds_write_barrier();  // B2'
    if (!SCORE) value_step(std::false_type{}, 0);
  }

  lds_write_barrier();
  float s0 = 0.f, s1 = 0.f;
  if (SCORE) {
    s0 = wave_sum_rows(l0);
    s1 = wave_sum_rows(l1);
    mx_mine[0] = s0;
    mx_mine[64] = s1;
  }
  lds_write_barrier();
  if (SCORE) {
    const float t0 = s0 + mx_part[0], t1 = s1 + mx_part[64];
    if (hh == 0) {
      al_row[0] = t0 > 0.f ? 1.0f / t0 : 0.f;
      al_row[64] = t1 > 0.f ? 1.0f / t1 : 0.f;
      if (g == 0) {
        if (x0.ok) a.lse[x0.qrow] = t0 > 0.f ? (m0 + fast_log2(t0)) * kLn2 : -INFINITY;
        if (x1.ok) a.lse[x1.qrow] = t1 > 0.f ? (m1 + fast_log2(t1)) * kLn2 : -INFINITY;
      }
    }
  }
  lds_write_barrier();
  if (!SCORE) store_rows(a, wt, L.al, o, lane, vq, block_rows);
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
  const int w = threadIdx.x >> 6;
  const int total_tiles = a.tile_cum[a.batch];
  const int block_rows = a.tok_per_tile * a.heads;
  const int row_blocks = (block_rows + kBlockRows - 1) / kBlockRows;
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) s_tile = atomicAdd(a.counter, 1);
    __syncthreads();
    const int t = s_tile;
    if (t >= total_tiles) break;
    const WorkTile wt = locate_work(a, t, row_blocks);
    if (w < 4)
      ws_codes_work_tile<true, CODE>(a, wt, L, w, lane, block_rows);
    else
      ws_codes_work_tile<false, CODE>(a, wt, L, w, lane, block_rows);
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
