// Device building blocks shared by the decode and prefill kernels (gfx950).
//
// A workgroup stages one 64-row cache page at a time in LDS and every wave
// attends its own 16 query rows against it:
//
//   S^T = K * Q^T     v_mfma_f32_16x16x32_bf16, A = K rows from LDS
//                     (16 tokens x 32 features per instruction), B = the
//                     wave's Q rows held in registers for the whole call
//   online softmax    in the S^T accumulator layout, each lane owns one
//                     query row and 16 of the page's 64 tokens, so the row
//                     max needs two cross-lane exchanges and the row sum
//                     none (it is reduced once, at the end)
//   O^T += V^T * P^T  A = V^T read with ds_read_b64_tr_b16 (the value
//                     columns are the first 512 columns of the same staged
//                     page), B = P^T taken straight from the S^T
//                     accumulators, so P never goes through LDS
//
// The O^T accumulators give each lane one query row and 4 consecutive value
// columns per 16-column tile, so the softmax rescale is a per-lane scalar.
//
// LDS layout of a staged page: row t starts at byte t * 1168 (the 1152-byte
// row plus one 16-byte pad).  The odd pitch (73 chunks) puts the 16 tokens
// one A-operand read touches, and the 4 tokens x 16 columns one transposed
// read touches, on distinct banks, while every LDS address stays an affine
// function of the loop indices, so it folds into the instructions'
// immediate offsets.  A page is exactly 73 wave-wide direct-to-LDS loads;
// the lanes that land on a pad slot re-read chunk 0 of their row.
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
constexpr int kLdsPitch = kRowBytes + 16;      // 1168: one row in LDS
constexpr int kLdsChunks = kLdsPitch / 16;     // 73
constexpr int kTileBytes = kPage * kLdsPitch;  // 74752: one staged page in LDS
constexpr int kTileLoads = kTileBytes / 1024;  // 73 wave-wide 16-byte loads per page
static_assert(kTileLoads * 1024 == kTileBytes, "a staged page is a whole number of wave loads");
constexpr int kQFrags = kDqk / 32;             // 18 k-steps of 32 features
constexpr int kOFrags = kDv / 16;              // 32 value-column tiles

// Byte offset of 16-byte chunk `chunk` of token `t` inside a staged page.
__device__ __forceinline__ int tile_off(int t, int chunk) { return t * kLdsPitch + chunk * 16; }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max_rows(float v) {
  // Max over the four lanes that hold the same query row (lane, lane^16, lane^32, lane^48).
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum_rows(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Global byte offset (within its page) that the lane's slot of wave-wide
// load i must fetch.  Rows at or past `valid` re-read row 0 of the same
// page, so the staged rows are always finite cache data and nothing past a
// request's length is ever read.
__device__ __forceinline__ int stage_src(int i, int lane, int valid) {
  const int s = i * 64 + lane;              // 16-byte slot in the staged page
  const int t = s / kLdsChunks;
  int c = s - t * kLdsChunks;
  c = c == kRowChunks ? 0 : c;              // pad slot
  const int ts = t < valid ? t : 0;
  return ts * kRowBytes + c * 16;
}

// Issue this wave's share (loads w, w + nwaves, ...) of the direct-to-LDS
// loads of one cache page into `stage`.
template <int NW>
__device__ __forceinline__ void stage_page(const uint8_t* __restrict__ page, MLA_LDS uint8_t* stage,
                                           int valid, int wave, int lane) {
  if (valid >= kPage) {
#pragma unroll
    for (int i0 = 0; i0 < kTileLoads; i0 += NW) {
      const int i = i0 + wave;
      if (NW * ((kTileLoads + NW - 1) / NW) == kTileLoads || i < kTileLoads)
        __builtin_amdgcn_global_load_lds((const void*)(page + stage_src(i, lane, kPage)),
                                         (MLA_LDS void*)(stage + i * 1024), 16, 0, 0);
    }
  } else {
    for (int i = wave; i < kTileLoads; i += NW)
      __builtin_amdgcn_global_load_lds((const void*)(page + stage_src(i, lane, valid)),
                                       (MLA_LDS void*)(stage + i * 1024), 16, 0, 0);
  }
}

// Per-wave attention state: 16 query rows, one per lane group position.
struct RowState {
  f32x4 o[kOFrags];  // O^T: lane holds row (lane & 15), columns 16*ct + 4*(lane>>4) + e
  float m;           // running max of scaled scores, log2 units (row-uniform)
  float l;           // this lane's share of the running sum
};

__device__ __forceinline__ void reset_state(RowState& st) {
#pragma unroll
  for (int i = 0; i < kOFrags; ++i) st.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
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

// Attend one staged page.  Token tt of the page is visible to this lane's
// row when tt <= lim (lim >= 63: whole page visible).
__device__ __forceinline__ void attend_page(const MLA_LDS uint8_t* tile, const bf16x8 (&qf)[kQFrags],
                                            int lim, float scale_log2, int lane, RowState& st) {
  const int r16 = lane & 15;
  const int g = lane >> 4;

  // ---- S^T = K Q^T for the page's 64 tokens (4 tiles of 16 tokens) ----
  // K fragments of k-step ks+1 are read while the MFMAs of k-step ks run.
  f32x4 acc[4];
  bf16x8 kc[4], kn[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    kc[mt] = lds_b128(tile + tile_off(16 * mt + r16, g));  // k-step 0
  }
#pragma unroll
  for (int ks = 0; ks < kQFrags; ++ks) {
    if (ks + 1 < kQFrags) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) kn[mt] = lds_b128(tile + tile_off(16 * mt + r16, 4 * (ks + 1) + g));
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma16x16x32(kc[mt], qf[ks], acc[mt]);
    if (ks + 1 < kQFrags) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) kc[mt] = kn[mt];
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- scale, mask, online softmax ----
  float s[16];
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tt = 16 * mt + 4 * g + e;
      float v = acc[mt][e] * scale_log2;
      v = tt <= lim ? v : -INFINITY;
      s[4 * mt + e] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = wave_max_rows(mx);
  // Raise the max only when the page's max exceeds it by more than the slack.
  const bool raise = mx > st.m + kRescaleSlack;
  if (__builtin_amdgcn_read_exec() & __ballot(raise)) {
    const float m_new = raise ? mx : st.m;
    const float alpha = fast_exp2(st.m - m_new);  // st.m = -inf: 0; unchanged rows: 1
    st.m = m_new;
    st.l *= alpha;
    // in groups, so that only a few accumulators are out of their registers at a time
#pragma unroll
    for (int c0 = 0; c0 < kOFrags; c0 += 4) {
#pragma unroll
      for (int ct = c0; ct < c0 + 4; ++ct) st.o[ct] *= alpha;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float m_use = st.m == -INFINITY ? 0.f : st.m;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i] = fast_exp2(s[i] - m_use);
    psum += s[i];
  }
  st.l += psum;
  bf16x8 pb[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pb[kk][e] = (__bf16)s[4 * (2 * kk) + e];
      pb[kk][4 + e] = (__bf16)s[4 * (2 * kk + 1) + e];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- O^T += V^T P^T: 2 k-steps of 32 tokens x 32 column tiles ----
  // Transposed reads: lane i of its 16-lane group supplies token
  // 32kk + 4g + i/4 (and that + 16) and columns 16ct + 4(i%4) .. +3, and
  // receives the 4 tokens of column 16ct + i.  Reads of step n+1 are issued
  // while the MFMA of step n runs.
  const int i16 = lane & 15;
  const int colq = 4 * (i16 & 3);
  const int tq = 4 * g + (i16 >> 2);
  const MLA_LDS uint8_t* vbase = tile + tq * kLdsPitch + colq * 2;
  auto v_addr = [&](int kk, int ct, int half) {
    return vbase + (32 * kk + 16 * half) * kLdsPitch + 32 * ct;
  };
  bf16x4 va0 = lds_tr16(v_addr(0, 0, 0)), va1 = lds_tr16(v_addr(0, 0, 1));
#pragma unroll
  for (int step = 0; step < 2 * kOFrags; ++step) {
    const int kk = step / kOFrags, ct = step % kOFrags;
    bf16x4 vn0, vn1;
    if (step + 1 < 2 * kOFrags) {
      const int kk1 = (step + 1) / kOFrags, ct1 = (step + 1) % kOFrags;
      vn0 = lds_tr16(v_addr(kk1, ct1, 0));
      vn1 = lds_tr16(v_addr(kk1, ct1, 1));
    }
    bf16x8 va;
    va[0] = va0[0]; va[1] = va0[1]; va[2] = va0[2]; va[3] = va0[3];
    va[4] = va1[0]; va[5] = va1[1]; va[6] = va1[2]; va[7] = va1[3];
    st.o[ct] = mfma16x16x32(va, pb[kk], st.o[ct]);
    if (step + 1 < 2 * kOFrags) {
      va0 = vn0;
      va1 = vn1;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Row totals at the end of a range: the row's full sum, 1/sum (0 when the
// row saw nothing), and the log-sum-exp in log2 units (-inf when empty).
__device__ __forceinline__ void finish_row(const RowState& st, float& inv, float& lse2) {
  const float l = wave_sum_rows(st.l);
  inv = l > 0.f ? 1.0f / l : 0.f;
  lse2 = l > 0.f ? st.m + fast_log2(l) : -INFINITY;
}

}  // namespace mla
