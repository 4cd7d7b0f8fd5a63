// The wave-specialised attention core shared by the prefill kernels and the
// INT8 / FP8 decode kernel (gfx950).
//
// A workgroup of eight waves attends one block of up to 64 query rows
// (four 16-row MFMA tiles) against staged 32-row tiles of its request's
// cache.  Waves 0-3 are score waves: score wave (rg, kh) holds the query
// fragments of rows 32 rg .. 32 rg + 31 and scores them against rows
// 16 kh .. 16 kh + 15 of each tile (each K fragment read from LDS feeds two
// MFMAs), then runs the online softmax of its half of the tile's rows and
// publishes the bf16 probabilities.  Waves 4-7 are value waves: value wave vq
// holds the accumulators of all 64 rows for value columns 128 vq ..
// 128 vq + 127 (each transposed V fragment read feeds four MFMAs).  Waves w
// and w + 4 share a SIMD.  The per-kernel pipelines (how the tiles reach LDS)
// are in the kernels' sources; this header holds the pieces they share and
// the INT8 / FP8 pipeline that both the prefill and the decode run.
#pragma once

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kPWin = 256;  // page ids staged per window (a pipeline restart per window)

// Waves that stage tiles (the value waves, the last four).
constexpr int kLoadWaves = 4;

// What every block needs of the call: the cache and its table, the score scale.
struct WsArgs {
  const uint8_t* kv;
  const float* kv_scale;
  const int32_t* page_table;
  int pt_stride;              // page-table entries per request
  int sub;                    // 64-row sub-pages per page
  float scale_log2;           // softmax_scale * log2(e)
};

// A block of up to 64 query rows of one request and the cache range it
// attends.  Row r of the block (0 .. 63) is row r0 + r of the request's rows
// (token-major: head h of the request's token i is row i * heads + h); it
// exists when r0 + r < nrows, its query is q[(r0 + r) * 576 ..], its output
// goes to out[(r0 + r) * 512 ..] and lse[r0 + r], and its token sees cache
// rows 0 .. vis0 + (r0 + r) / heads.
struct WsBlock {
  const uint16_t* q;          // bf16 query rows of the request, row 0
  uint16_t* out;              // bf16 output rows (normalised), row 0
  float* lse;                 // log-sum-exp of row 0
  float lse_mul;              // ln 2 for the natural-log LSE of a final output, 1 for a log2 partial
  int r0;                     // first row of the block
  int nrows;                  // rows of the request
  int vis0;                   // last cache row seen by row 0's token
  int heads;
  int b;                      // request (row of the page table)
  int p_lo, p_hi;             // 64-row sub-pages [p_lo, p_hi) to attend
  int kv_end;                 // cached rows of the request: none at or past it is read
};

// The block is the same for every lane; the compiler cannot always prove it
// (fields read back from LDS or chosen per segment), and then it holds them
// in vector registers that the core needs.  readfirstlane moves each field to
// a scalar register.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ WsBlock wave_uniform(const WsBlock& k) {
  WsBlock u;
  u.q = wave_uniform(k.q);
  u.out = wave_uniform(k.out);
  u.lse = wave_uniform(k.lse);
  u.lse_mul = __builtin_bit_cast(float, wave_uniform(__builtin_bit_cast(int, k.lse_mul)));
  u.r0 = wave_uniform(k.r0);
  u.nrows = wave_uniform(k.nrows);
  u.vis0 = wave_uniform(k.vis0);
  u.heads = wave_uniform(k.heads);
  u.b = wave_uniform(k.b);
  u.p_lo = wave_uniform(k.p_lo);
  u.p_hi = wave_uniform(k.p_hi);
  u.kv_end = wave_uniform(k.kv_end);
  return u;
}

// A query row of a block: exists?, its index from the request's row 0, the
// last cache row its token sees.
struct QRow {
  bool ok;
  int qrow;
  int vis_last;
};

__device__ __forceinline__ QRow ws_row(const WsBlock& k, int r) {
  QRow x;
  x.qrow = k.r0 + r;
  x.ok = x.qrow < k.nrows;
  x.vis_last = k.vis0 + x.qrow / k.heads;
  return x;
}

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


// Value waves, at the end of a block: normalise (al holds 1 / row sum) and
// store the wave's 128 columns of each of the block's rows.
__device__ __forceinline__ void ws_store_rows(const WsBlock& k, const MLA_LDS float* al,
                                              const f32x4 (&o)[kVQTiles][kVCTiles], int lane, int vq) {
  const int col = 128 * vq + 4 * (lane >> 4);
#pragma unroll
  for (int qt = 0; qt < kVQTiles; ++qt) {
    const QRow x = ws_row(k, 16 * qt + (lane & 15));
    const float inv = al[64 * qt + lane];
    if (x.ok) {
      uint16_t* dst = k.out + (size_t)x.qrow * kDv + col;
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

// ---------------------------------------------------------------------------
// INT8 / FP8 cache (CODE), K prefetch depth KAHEAD (the score waves here
// also hold the row scales).  Both wave kinds bring their share of each
// tile's codes (see CodeRegs below; the value threads also the 32 row
// scales) straight into registers with ordinary global loads, a step ahead,
// and widen them to exact bf16 into one of three converted tiles in LDS (the
// tile's 32 row scales beside it).  No code byte passes through LDS.  Step k:
//  - B1(k): tile k is converted (in step k - 1);
//  - score waves: softmax of tile k - 1 (probabilities times their row's
//    scale, selected to 0 on masked rows so that a non-finite scale there
//    cannot leak; the row sums take the unscaled probabilities), then the
//    scores of tile k from its converted tile, each row's score times its
//    scale; value waves: the conversion of their part of tile k + 1 (its
//    codes were requested in step k - 1) and the loads of their part of
//    tile k + 2 into the registers that just freed up;
//  - B2(k): the probabilities of tile k - 1 are published;
//  - score waves: the same for their part of tiles k + 1 and k + 2; value
//    waves: the value product of tile k - 1, re-reading each V fragment
//    from tile k's converted tile behind its four MFMAs.
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

// K fragments the score waves read ahead of their MFMAs: 4 measured best on
// the INT8 and FP8 prefill and the FP8 decode, 3 on the INT8 decode (67.7
// against 69.6 us on the 4 x 64K shape, 399 against 403 us on 8 x 256K; 3 costs
// the FP8 prefill 8%, and 5 or 6 were slower everywhere).
constexpr int kKAheadC = 4;
constexpr int kKAheadDecodeInt8 = 3;

// Each tile row's 72 units of 8 codes are split between the two wave kinds:
// value thread t (0..255) holds units kVUnits (t & 7) .. + kVUnits - 1 of tile
// row t / 8 (and, for t < 32, row t's scale); score thread t holds units
// 8 kVUnits + kSUnits (t & 7) .. + kSUnits - 1.  The value waves widen their
// part in the score phase, the score waves theirs after B2, where they would
// otherwise wait for the value product.
constexpr int kCodeUnits = kI8RowBytes / 8 / 8;  // 9 units of 8 codes per thread and row
constexpr int kVUnits = 6;
constexpr int kSUnits = kCodeUnits - kVUnits;

template <int N>
struct CodeRegs {
  u32x2 c[N];
  float sc;  // value threads 0 .. 31: row scale of tile row `thread`
};

// Request this thread's N units (from unit u0 + N (t & 7) of tile row t / 8)
// of tile `half` (rows 32 half ..) of a page; rows at or past `rem` re-read
// row 0's codes, and their scales are read as they are and never used
// unmasked.  SCALE: also the row scale (threads t < 32).
template <int N, bool SCALE>
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ page, const float* __restrict__ spage,
                                           int half, int rem, int t, int u0, CodeRegs<N>& r) {
  const int row = kTileRows * half + (t >> 3);
  const uint8_t* src = page + (size_t)(row < rem ? row : 0) * kI8RowBytes + 8 * (u0 + N * (t & 7));
#pragma unroll
  for (int i = 0; i < N; ++i) r.c[i] = *reinterpret_cast<const u32x2*>(src + 8 * i);
  if constexpr (SCALE) r.sc = t < kTileRows ? spage[kTileRows * half + t] : 0.f;
}

// Widen this thread's units into a converted tile (pitch 1184, like a staged
// bf16 tile) and (SCALE) the row scales into `tsc`.
template <int CODE, int N, bool SCALE>
__device__ __forceinline__ void store_codes(const CodeRegs<N>& r, MLA_LDS uint8_t* cvt, MLA_LDS float* tsc, int t,
                                            int u0) {
  MLA_LDS uint8_t* dst = cvt + (t >> 3) * kLdsPitch + 16 * (u0 + N * (t & 7));
#pragma unroll
  for (int i = 0; i < N; ++i) {
    u32x4 o;
    o[0] = codepair_to_bf16<CODE, 0>(r.c[i][0]); o[1] = codepair_to_bf16<CODE, 1>(r.c[i][0]);
    o[2] = codepair_to_bf16<CODE, 0>(r.c[i][1]); o[3] = codepair_to_bf16<CODE, 1>(r.c[i][1]);
    *reinterpret_cast<MLA_LDS u32x4*>(dst + 16 * i) = o;
  }
  if constexpr (SCALE) {
    if (t < kTileRows) tsc[t] = r.sc;
  }
}

struct WsCodesLds {
  MLA_LDS uint8_t* cvt;  // three converted tiles (bf16, pitch 1184)
  MLA_LDS float* tsc;    // their row scales, 32 each
  MLA_LDS float* mx;
  MLA_LDS uint8_t* pb;
  MLA_LDS float* al;
  int* pid;
};

// One block of up to 64 query rows against sub-pages [p_lo, p_hi) of its
// request, INT8 / FP8 cache (see above), as a score wave (SCORE) or a value
// wave: both kinds pass the same barriers in the same order.
template <bool SCORE, int CODE, int KAHEAD = kKAheadC>
__device__ __forceinline__ void ws_codes_range(const WsArgs& a, const WsBlock& k_, const WsCodesLds& L, int w,
                                               int lane) {
  const int rg = (w & 3) >> 1;  // score waves: row group
  const int hh = w & 1;         // score waves: tile-row half kh
  const int vq = w & 3;         // value waves: column quarter
  const int vt = threadIdx.x - (kWaves - kLoadWaves) * 64;  // value waves: thread 0 .. 255
  const int g = lane >> 4;
  const int r0 = 32 * rg + (lane & 15);
  const QRow x0 = ws_row(k_, r0), x1 = ws_row(k_, r0 + 16);
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
  CodeRegs<kVUnits> rc;  // value waves: their codes of the next tile to convert
  CodeRegs<kSUnits> rs;  // score waves: theirs
  if (SCORE) {
    issue_q(x0.ok ? k_.q + (size_t)x0.qrow * kDqk : nullptr, lane, q0);
    issue_q(x1.ok ? k_.q + (size_t)x1.qrow * kDqk : nullptr, lane, q1);
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
    bf16x8 kb[KAHEAD];
    if constexpr (kScores) {
#pragma unroll
      for (int d = 0; d < KAHEAD; ++d) kb[d] = lds_b128(kbase + 64 * d);
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
        const bf16x8 kf = kb[ks % KAHEAD];
        if (ks + KAHEAD < kQFrags) kb[ks % KAHEAD] = lds_b128(kbase + 64 * (ks + KAHEAD));
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

  for (int plo = k_.p_lo; plo < k_.p_hi; plo += kPWin) {
    const int n = min(kPWin, k_.p_hi - plo);
    lds_barrier();  // the previous window's page ids and converted tiles are no longer read
    for (int k = threadIdx.x; k < n; k += kWaves * 64)
      L.pid[k] = sub_page(a.page_table, (size_t)k_.b * a.pt_stride, plo + k, a.sub);
    __builtin_amdgcn_s_waitcnt(0);  // the page ids are in LDS
    lds_barrier();
    const int ntiles = min(2 * n, (k_.kv_end - kPage * plo + kTileRows - 1) / kTileRows);
    auto lim_of = [&](const QRow& x, int k) { return x.ok ? x.vis_last - (kPage * plo + kTileRows * k) : -1; };
    // this thread's codes of tile k (tiles past the window's last re-read the
    // last one, so that the registers always hold defined data; they are
    // converted into a buffer nobody reads)
    auto load = [&](int k) {
      const int kk = min(k, ntiles - 1);
      const int p = kk >> 1;
      const int pid = L.pid[p];
      const uint8_t* page = a.kv + (size_t)pid * kI8PageBytes;
      const float* spage = a.kv_scale + (size_t)pid * kPage;
      const int rem = k_.kv_end - kPage * (plo + p);
      if constexpr (SCORE)
        load_codes<kSUnits, false>(page, spage, kk & 1, rem, threadIdx.x, 8 * kVUnits, rs);
      else
        load_codes<kVUnits, true>(page, spage, kk & 1, rem, vt, 0, rc);
    };
    auto convert = [&](int k) {
      if constexpr (SCORE)
        store_codes<CODE, kSUnits, false>(rs, cvt_of(k), tsc_of(k), threadIdx.x, 8 * kVUnits);
      else
        store_codes<CODE, kVUnits, true>(rc, cvt_of(k), tsc_of(k), vt, 0);
    };
    auto value_step = [&](auto refill, int next) {
      value_product<decltype(refill)::value>(L.pb, L.al, vb, o, cvt_of(next), lane, vq);
    };
    // steps k >= 1; the registers hold this thread's codes of tile k + 1
    auto step = [&](int k) {
      lds_write_barrier();  // B1(k): tile k converted
      if (SCORE) {
        score_step(std::true_type{}, k, k - 1, lim_of(x0, k), lim_of(x1, k));
      } else {
        convert(k + 1);
        load(k + 2);
      }
      lds_write_barrier();  // B2(k): the probabilities of tile k - 1 are published
      if (SCORE) {
        mx_mine[0] = mx0;
        mx_mine[64] = mx1;
        convert(k + 1);
        load(k + 2);
      } else {
        value_step(std::true_type{}, k);  // tile k - 1, then V of tile k into vb
      }
    };

    load(0);
    convert(0);
    load(1);
    lds_write_barrier();  // B1(0): tile 0 converted
    if (SCORE) score_tile(0, lim_of(x0, 0), lim_of(x1, 0));
    lds_write_barrier();  // B2(0)
    if (SCORE) {
      mx_mine[0] = mx0;
      mx_mine[64] = mx1;
    }
    convert(1);
    load(2);
    if (!SCORE) values_fetch(cvt_of(0), lane, vq, vb);  // V of tile 0
    for (int k = 1; k < ntiles; ++k) step(k);
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
        if (x0.ok) k_.lse[x0.qrow] = t0 > 0.f ? (m0 + fast_log2(t0)) * k_.lse_mul : -INFINITY;
        if (x1.ok) k_.lse[x1.qrow] = t1 > 0.f ? (m1 + fast_log2(t1)) * k_.lse_mul : -INFINITY;
      }
    }
  }
  lds_write_barrier();
  if (!SCORE) ws_store_rows(k_, L.al, o, lane, vq);
}

}  // namespace mla
