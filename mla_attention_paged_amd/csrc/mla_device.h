// Device building blocks shared by the decode and prefill kernels (gfx950).
//
// A workgroup of eight waves (two per SIMD: waves w and w + 4 share one)
// attends a block of up to 64 query rows against the cache, which it
// streams through a ring of LDS stages of 32 cache rows (half a page) each
// (three stages in the bf16 decode kernel, four in the bf16 prefill kernel,
// three converted tiles in the INT8 / FP8 kernels).  In the bf16 decode
// kernel, waves w and w + 4 share the 16 query rows 16 (w % 4) .. +15 and
// split the work of each tile in two halves, h = w / 4 (the prefill kernels
// and the INT8 / FP8 decode kernel specialise their waves instead: score
// waves and value waves, in mla_ws.h):
//
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16 over the 576 features: A = 16
//                   cache rows (rows 16h .. 16h + 15 of the tile) read from
//                   LDS, B = the wave's Q rows, held in registers for the
//                   whole range
//   exchange        each wave hands its 16 x 16 score block to its partner
//                   through LDS, so both hold the row's scores for all 32
//                   rows of the tile
//   online softmax  identical in both waves: each lane owns one query row
//                   and 8 of the 32 rows, so the row max needs two lane
//                   swaps and the row sum none (it is reduced at the end)
//   O^T += V^T P^T  A = V^T read with ds_read_b64_tr_b16 (the value columns
//                   are the first 512 columns of the same staged rows), B =
//                   P^T taken straight from the score registers; wave half h
//                   accumulates value columns 256h .. 256h + 255
//
// Splitting the value columns halves the accumulators (64 registers), which
// is what lets two waves share a SIMD and hide each other's softmax, LDS and
// barrier latency behind their MFMAs; splitting the score rows keeps the
// total MFMA and LDS work per tile the same as with one wave per 16 rows.
//
// LDS layout of a staged tile: row t starts at byte t * 1184 (the 1152-byte
// row plus 32 bytes of pad; 296 dwords, an odd multiple of 8 modulo the 64
// banks).  Measured on gfx950, this pitch serves both read shapes near the
// LDS peak: the A-operand reads of 16 rows x 16 bytes (~220 B/clk/CU) and
// the transposed reads of 16 rows x 32 bytes (~145 B/clk/CU), against ~120
// for a 1168-byte pitch and ~60 for the unpadded 1152.  Every LDS address
// stays an affine function of the loop indices, so it folds into the
// instructions' immediate offsets.  A tile is exactly 37 wave-wide
// direct-to-LDS loads; the lanes that land on a pad slot re-read chunk 0 of
// their row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr int kRowBytes = kDqk * 2;            // 1152: one cache row in HBM
constexpr int kRowChunks = kRowBytes / 16;     // 72
constexpr int kPageBytes = kPage * kRowBytes;  // 73728: one page in HBM
constexpr int kLdsPitch = kRowBytes + 32;      // 1184: one row in LDS
constexpr int kLdsChunks = kLdsPitch / 16;     // 74
constexpr int kTileRows = 32;                  // rows per LDS stage (half a page)
constexpr int kTileSlots = kTileRows * kLdsChunks;      // 2368 16-byte slots
constexpr int kStageLoads = kTileSlots / 64;            // 37 wave-wide loads per tile
static_assert(kStageLoads * 64 == kTileSlots, "a tile is a whole number of wave-wide loads");
constexpr int kStageBytes = kStageLoads * 1024;         // 37888

// INT8 / FP8 cache: a row is 576 one-byte codes (and one fp32 scale beside the
// page); a 32-row tile of codes is 18,432 contiguous bytes of its page.
constexpr int kI8RowBytes = kDqk;                          // 576
constexpr int kI8PageBytes = kPage * kI8RowBytes;          // 36864
constexpr int kI8CodeBytes = kTileRows * kI8RowBytes;      // 18432
constexpr int kQFrags = kDqk / 32;             // 18 k-steps of 32 features
constexpr int kOFrags = kDv / 16;              // 32 value-column tiles
constexpr int kWaves = 8;                      // waves per workgroup (two per SIMD)
constexpr int kBlockRows = kBlockRowsHost;     // query rows per workgroup (64)
constexpr int kOHalf = kOFrags / 2;            // value-column tiles per wave

// Pages of sub * 64 rows are laid out as sub consecutive 64-row sub-pages,
// so the kernels walk the cache in 64-row sub-pages: logical sub-page j of
// the request whose page-table row starts at `row` is sub-page
// (entry j / sub) * sub + j % sub of the cache.
__device__ __forceinline__ int sub_page(const int32_t* __restrict__ page_table, size_t row, int j, int sub) {
  if (sub == 1) return page_table[row + j];
  const int e = j / sub;
  return page_table[row + e] * sub + (j - e * sub);
}

// Byte offset of 16-byte chunk `chunk` of token `t` inside a staged page.
__device__ __forceinline__ int tile_off(int t, int chunk) { return t * kLdsPitch + chunk * 16; }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left free), GFX9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Direct-to-LDS loads wave w issues per tile when LOADS are spread over NW
// waves (load i is issued by wave i % NW).
template <int NW, int LOADS = kStageLoads>
__device__ __forceinline__ constexpr int stage_loads_of(int w) { return (LOADS - w + NW - 1) / NW; }

// Wait until this wave's loads of the oldest outstanding tile have landed,
// leaving the loads of `ahead` (0..4) younger tiles in flight.
template <int NW, int LOADS = kStageLoads>
__device__ __forceinline__ void wait_tile(int ahead, int w) {
  constexpr int hi = stage_loads_of<NW, LOADS>(0);
  constexpr int lo = stage_loads_of<NW, LOADS>(NW - 1);
  const bool big = stage_loads_of<NW, LOADS>(w) == hi;
  switch (ahead) {
    case 4: if (big) wait_vmcnt<4 * hi>(); else wait_vmcnt<4 * lo>(); break;
    case 3: if (big) wait_vmcnt<3 * hi>(); else wait_vmcnt<3 * lo>(); break;
    case 2: if (big) wait_vmcnt<2 * hi>(); else wait_vmcnt<2 * lo>(); break;
    case 1: if (big) wait_vmcnt<hi>(); else wait_vmcnt<lo>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// Workgroup barrier that is also a compiler memory barrier, without the
// vmcnt(0) that a full fence would add (it would drain the load ring).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Same, after this wave's own LDS writes have completed.
__device__ __forceinline__ void lds_write_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reductions over the four lanes that hold the same query row (lane,
// lane^16, lane^32, lane^48), with the gfx950 row-swap permutes (VALU only,
// no LDS round trip).  Each swap returns the lane's own value and its
// partner's in some order; max and sum of the pair are symmetric, so the
// result is the same whichever output holds which, and it is bitwise equal
// on all four lanes.
__device__ __forceinline__ float pair_max(float v, bool x32) {
  const unsigned u = __float_as_uint(v);
  const auto r = x32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float v, bool x32) {
  const unsigned u = __float_as_uint(v);
  const auto r = x32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max_rows(float v) { return pair_max(pair_max(v, false), true); }
__device__ __forceinline__ float wave_sum_rows(float v) { return pair_sum(pair_sum(v, false), true); }

// Global byte offset (within its page) that the lane's slot of wave-wide
// load i of tile `half` (0: rows 0-31 of the page, 1: rows 32-63) fetches.
// Rows at or past `rem` (the request's rows from the page start) re-read row
// 0 of the page, so the staged rows are always finite cache data and nothing
// past a request's length is ever read.
__device__ __forceinline__ int stage_src(int i, int lane, int half, int rem) {
  const int s = i * 64 + lane;              // 16-byte slot in the stage
  const int t = s / kLdsChunks;             // 0..31
  int c = s - t * kLdsChunks;
  c = c >= kRowChunks ? 0 : c;              // pad slots
  const int row = kTileRows * half + t;
  const int src = row < rem ? row : 0;
  return src * kRowBytes + c * 16;
}

// One wave-wide direct-to-LDS load: lane l's 16 bytes at base + voff land at
// LDS byte lds + 16 l.  Issued as inline assembly so that the compiler does
// not track it: its alias analysis cannot tell ring stages apart and would
// otherwise wait for every in-flight stage before each LDS read.  The
// kernels synchronise the ring themselves (wait_tile + s_barrier).  M0 holds
// the LDS address.  Wait states: a vector memory instruction that reads an
// SGPR a VALU instruction wrote needs five (the compiler often writes the
// base address with v_readfirstlane right before this block, and it does not
// pad inline assembly for that hazard): the leading s_nop 2 gives three, the
// M0 write and the s_nop 0 behind it (the M0-write hazard of an LDS load)
// two more.
__device__ __forceinline__ void lds_dma16(const uint8_t* base, int voff, const MLA_LDS uint8_t* lds) {
  // Both scalar operands are wave-uniform; readfirstlane makes that explicit
  // so that they are allocated to SGPRs.
  // (readfirstlane returns int: go through uint32_t so that neither half is
  // sign-extended when the 64-bit address is reassembled)
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t b_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t b_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t bs = ((uint64_t)b_hi << 32) | (uint64_t)b_lo;
  asm volatile("s_nop 2\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m), "v"(voff), "s"(bs)
               : "memory");
}

// Issue this wave's share (loads w, w + NW, ...) of the direct-to-LDS loads
// of one tile into `stage`.
template <int NW>
__device__ __forceinline__ void stage_tile(const uint8_t* __restrict__ page, int half, int rem,
                                           MLA_LDS uint8_t* stage, int wave, int lane) {
#pragma unroll
  for (int i0 = 0; i0 < kStageLoads; i0 += NW) {
    const int i = i0 + wave;
    if (i < kStageLoads) lds_dma16(page, stage_src(i, lane, half, rem), stage + i * 1024);
  }
}

// Two signed int8 codes (bytes 2k, 2k+1 of x) as two exact bf16 values.
__device__ __forceinline__ unsigned i8pair_to_bf16(unsigned x, int k) {
  const float f0 = (float)(int)(signed char)(x >> (16 * k));
  const float f1 = (float)(int)(signed char)(x >> (16 * k + 8));
  // small integers: the upper 16 bits of the fp32 value are the exact bf16
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

// Two E4M3 codes (bytes 2k, 2k+1 of x) as two exact bf16 values, in one
// gfx950 scaled FP8 -> bf16 conversion with scale 1 (it decodes the OCP E4M3
// format; every code byte is checked on the GPU through both attention
// kernels).  E4M3 values have 4 significant bits and exponents inside bf16's
// normal range, so the result is exact.
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
template <int K>
__device__ __forceinline__ unsigned fp8pair_to_bf16(unsigned x) {
  const bf16x2_cvt b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, K != 0);
  return __builtin_bit_cast(unsigned, b);
}

// Cache code formats of the scaled caches.
constexpr int kCodeInt8 = 1;
constexpr int kCodeFp8 = 2;

template <int CODE, int K>
__device__ __forceinline__ unsigned codepair_to_bf16(unsigned x) {
  return CODE == kCodeFp8 ? fp8pair_to_bf16<K>(x) : i8pair_to_bf16(x, K);
}

// Per-wave attention state: 16 query rows x 256 value columns.
struct RowState {
  f32x4 o[kOHalf];   // O^T: lane holds row (lane & 15), columns 256h + 16ct + 4(lane>>4) + e
  float m;           // running max of scaled scores, log2 units (row-uniform)
  float l;           // this lane's share of the running sum
};

__device__ __forceinline__ void reset_state(RowState& st) {
#pragma unroll
  for (int i = 0; i < kOHalf; ++i) st.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Start loading this wave's Q fragments (no wait; see load_q).
__device__ __forceinline__ void issue_q(const uint16_t* __restrict__ qrow, int lane, bf16x8 (&qf)[kQFrags]) {
  const int g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < kQFrags; ++ks)
    qf[ks] = qrow ? *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g) : bf16x8{};
}

// Load this wave's Q fragments: lane holds row (lane & 15), features
// 32*ks + 8*(lane>>4) .. +7 for each k-step ks.  `qrow` is null for rows
// past the end of the block (they attend with a zero query and are never
// written).
__device__ __forceinline__ void load_q(const uint16_t* __restrict__ qrow, int lane, bf16x8 (&qf)[kQFrags]) {
  const int g = lane >> 4;
  if (qrow) {
#pragma unroll
    for (int ks = 0; ks < kQFrags; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g);
  } else {
#pragma unroll
    for (int ks = 0; ks < kQFrags; ++ks) qf[ks] = bf16x8{};
  }
  // Settle the Q loads here: otherwise the tile loop, whose in-flight load
  // count the compiler cannot track, would wait for every load before each tile.
  wait_vmcnt<0>();
}

// A workgroup's 64-row query block staged in LDS: row r's 16-byte chunk c
// sits in slot 72 r + (c ^ ((r >> 1) & 7)).  The XOR keeps c inside its
// group of eight chunks; it spreads the 16 rows of one fragment read over
// all 16 bank groups (the unswizzled 1152-byte pitch puts every other row
// on the same banks).
constexpr int kQLoads = kBlockRows * kRowChunks / 64;  // 72 wave-wide loads

__device__ __forceinline__ int q_slot(int r, int c) { return kRowChunks * r + (c ^ ((r >> 1) & 7)); }

// Issue loads i = first, first + step, ... of the block's direct-to-LDS
// loads that hold rows 0 .. nrows - 1 of `qblk` (1 <= nrows <= 64), in whole
// 1 KB wave loads.  Slots of the last load past row nrows - 1 repeat it, so
// nothing past the block's rows is read; later rows stay unwritten (their
// fragments are zeroed on reading).
__device__ __forceinline__ void stage_q(const uint16_t* __restrict__ qblk, int nrows, MLA_LDS uint8_t* dst,
                                        int first, int step, int lane) {
  const int loads = (nrows * kRowChunks + 63) / 64;
  for (int i = first; i < loads; i += step) {
    const int sl = i * 64 + lane;
    const int r = sl / kRowChunks;
    const int c = (sl - r * kRowChunks) ^ ((r >> 1) & 7);
    lds_dma16(reinterpret_cast<const uint8_t*>(qblk), (r < nrows ? r : nrows - 1) * kRowBytes + c * 16,
              dst + i * 1024);
  }
}

// This wave's Q fragments (block rows 16 rg .. 16 rg + 15, the layout of
// load_q) from a staged block; zero where `ok` is false.
__device__ __forceinline__ void read_q(const MLA_LDS uint8_t* src, int rg, int lane, bool ok,
                                       bf16x8 (&qf)[kQFrags]) {
  const int r = 16 * rg + (lane & 15);
  const int g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < kQFrags; ++ks)
    qf[ks] = ok ? *reinterpret_cast<const MLA_LDS bf16x8*>(src + 16 * q_slot(r, 4 * ks + g)) : bf16x8{};
}

// Scores may run this far (log2 units) above the running max before the
// max is raised and the accumulators rescaled.  The result is the same (the
// final normalisation uses the same stale max); it only bounds the
// probabilities by 2^kRescaleSlack, far inside fp32 and bf16 range, and lets
// almost every page skip the 128-register rescale.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ bf16x8 lds_b128(const MLA_LDS uint8_t* p) {
  return *reinterpret_cast<const MLA_LDS bf16x8*>(p);
}

__device__ __forceinline__ bf16x4 lds_tr16(const MLA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p));
}

// LDS read prefetch distances (in MFMA steps) of the two contractions.
constexpr int kKDepth = 3;
constexpr int kVDepth = 3;

// ---------------------------------------------------------------------------
// Pipelined core (bf16 cache).  A wave's work on a tile is split into three
// parts so that consecutive tiles overlap: while the score MFMAs of tile k
// run, the same wave's VALU performs the softmax of tile k-1, and the value
// product of tile k-1 follows.  Two tiles are resident (k-1 for values, k for
// scores) and one is loading, so the ring has three stages; one 37 KB tile
// in flight per CU already saturates HBM on gfx950 (measured: ~5.7 TB/s).
// ---------------------------------------------------------------------------
constexpr int kPStages = 3;

// Scores of this wave's 16 rows of the tile against its 16 query rows: the
// 18 k-steps alternate between two accumulators (two independent MFMA
// chains), summed at the end.
__device__ __forceinline__ f32x4 tile_scores(const MLA_LDS uint8_t* tile, const bf16x8 (&qf)[kQFrags],
                                             int lane, int half) {
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const MLA_LDS uint8_t* kbase = tile + tile_off(16 * half + r16, g);
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  bf16x8 kb[kKDepth + 1];
#pragma unroll
  for (int d = 0; d < kKDepth; ++d) kb[d] = lds_b128(kbase + 64 * d);
#pragma unroll
  for (int ks = 0; ks < kQFrags; ++ks) {
    if (ks + kKDepth < kQFrags) kb[(ks + kKDepth) % (kKDepth + 1)] = lds_b128(kbase + 64 * (ks + kKDepth));
    if (ks & 1)
      a1 = mfma16x16x32(kb[ks % (kKDepth + 1)], qf[ks], a1);
    else
      a0 = mfma16x16x32(kb[ks % (kKDepth + 1)], qf[ks], a0);
  }
  return a0 + a1;
}

// Online softmax of one tile from the two score halves (lo: tile rows
// 4g + e, hi: 16 + 4g + e), bitwise identical in both partner waves.  The
// running max and sum are updated here; the factor alpha by which the value
// accumulators must be rescaled is returned and applied by the caller
// (rescale_o), only when some row's max was raised, so that this code stays
// one branch-free block that can be interleaved with the next tile's score
// MFMAs.  Returns the probabilities in the B-operand layout of the value
// product.
__device__ __forceinline__ bf16x8 tile_softmax(f32x4 lo, f32x4 hi, int lim, float scale_log2, int lane,
                                               RowState& st, float& alpha) {
  const int g = lane >> 4;
  float s[8];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v0 = 4 * g + e <= lim ? lo[e] * scale_log2 : -INFINITY;
    const float v1 = 16 + 4 * g + e <= lim ? hi[e] * scale_log2 : -INFINITY;
    s[e] = v0;
    s[4 + e] = v1;
    mx = fmaxf(mx, fmaxf(v0, v1));
  }
  mx = wave_max_rows(mx);
  const float m_new = mx > st.m + kRescaleSlack ? mx : st.m;
  // unchanged max: exactly 1 (also when both are -inf); first finite max: 0
  alpha = m_new == st.m ? 1.f : fast_exp2(st.m - m_new);
  st.m = m_new;
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[i] = fast_exp2(s[i] - m_use);
    psum += s[i];
  }
  st.l = st.l * alpha + psum;
  bf16x8 pb;
#pragma unroll
  for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[e];
  return pb;
}

// Apply a raised max to the value accumulators; skipped (uniform branch)
// when no row of the wave changed its max, the common case after the first
// tiles of a range.
__device__ __forceinline__ void rescale_o(RowState& st, float alpha) {
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int ct = 0; ct < kOHalf; ++ct) st.o[ct] *= alpha;
  }
}

// Value product of one tile for this wave's 256 value columns.
__device__ __forceinline__ void tile_values(const MLA_LDS uint8_t* tile, bf16x8 pb, int lane, int half,
                                            RowState& st) {
  const int g = lane >> 4;
  const int i16 = lane & 15;
  const int colq = 4 * (i16 & 3);
  const int tq = 4 * g + (i16 >> 2);
  const MLA_LDS uint8_t* vbase = tile + tq * kLdsPitch + colq * 2 + 512 * half;
  bf16x4 vb[kVDepth + 1][2];
#pragma unroll
  for (int d = 0; d < kVDepth; ++d) {
    vb[d][0] = lds_tr16(vbase + 32 * d);
    vb[d][1] = lds_tr16(vbase + 16 * kLdsPitch + 32 * d);
  }
#pragma unroll
  for (int ct = 0; ct < kOHalf; ++ct) {
    if (ct + kVDepth < kOHalf) {
      vb[(ct + kVDepth) % (kVDepth + 1)][0] = lds_tr16(vbase + 32 * (ct + kVDepth));
      vb[(ct + kVDepth) % (kVDepth + 1)][1] = lds_tr16(vbase + 16 * kLdsPitch + 32 * (ct + kVDepth));
    }
    const bf16x4 v0 = vb[ct % (kVDepth + 1)][0], v1 = vb[ct % (kVDepth + 1)][1];
    bf16x8 va;
    va[0] = v0[0]; va[1] = v0[1]; va[2] = v0[2]; va[3] = v0[3];
    va[4] = v1[0]; va[5] = v1[1]; va[6] = v1[2]; va[7] = v1[3];
    st.o[ct] = mfma16x16x32(va, pb, st.o[ct]);
  }
}

// Steady-state step of the pipeline: scores of tile k (returned) with the
// softmax of tile k-1 interleaved into the MFMA chain, then the value
// product of tile k-1.  Scores and softmax are independent and in one
// basic block, so the VALU work can issue while the MFMAs execute.
__device__ __forceinline__ f32x4 tile_step(const MLA_LDS uint8_t* tile_k, const MLA_LDS uint8_t* tile_prev,
                                           const bf16x8 (&qf)[kQFrags], f32x4 lo, f32x4 hi, int lim,
                                           float scale_log2, int lane, int half, RowState& st) {
  const f32x4 sc = tile_scores(tile_k, qf, lane, half);
  float alpha;
  const bf16x8 pb = tile_softmax(lo, hi, lim, scale_log2, lane, st, alpha);
  rescale_o(st, alpha);
  tile_values(tile_prev, pb, lane, half, st);
  return sc;
}

// Row totals at the end of a range: the row's full sum, 1/sum (0 when the
// row saw nothing), and the log-sum-exp in log2 units (-inf when empty).
__device__ __forceinline__ void finish_row(const RowState& st, float& inv, float& lse2) {
  const float l = wave_sum_rows(st.l);
  inv = l > 0.f ? 1.0f / l : 0.f;
  lse2 = l > 0.f ? st.m + fast_log2(l) : -INFINITY;
}

}  // namespace mla
