// Query absorption and value up-projection: the per-head products on either
// side of the latent attention, as batched bf16 GEMMs on MFMA.
//
// Sources: [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎", section
// "Kernel：让 MLA 真正跑满 GPU" (attention over compressed latent rows; query x
// latent key is decode's first product), and the published MLA formulation
// [MLA] (DeepSeek-V2, arXiv:2405.04434) for the absorbed form: per head h,
// q_abs = W_UK[h]^T q_nope (512 values from 128) ahead of the attention, and
// the head output W_UV[h] o_lat (128 values from 512) after it.
//
// Both are C[m][n] = sum_k A[m][k] Bt[n][k] per head ("NT"): A's rows are the
// tokens' per-head vectors, Bt's rows the weight's output index, both
// contiguous in k.  The caller passes W_UK[h] transposed ([512][128]) for that
// reason; W_UV[h] ([128][512]) already is.  The work is memory-bound (85 flop
// per byte at the absorption's shape), so the kernel is shaped around the
// bytes.  A workgroup owns one head and a contiguous range of token blocks;
// its four waves split the N output columns, and each wave loads its slice of
// the weight (N/4 rows x K: 128 registers per lane at both shapes) into
// registers once and keeps it for every token block of the range, so the
// weights are read from memory once per range, not once per block (measured:
// with the weight fragments re-read from L2 for every 64-token block, the
// weight loads alone took 20 / 28 of the 62 / 59 us of the two products).  Per
// block of 16 TT tokens: A fragments (from global memory, or staged once in
// LDS when K = 512), v_mfma_f32_16x16x32_bf16 with the weight fragment as A
// operand (D = Bt A^T: each lane holds four consecutive output columns of one
// token), then the tile goes through LDS so that the stores write whole
// 128-byte lines.  fp32 accumulation, bf16 output rounded to nearest even.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

// A_LDS: the block's A tile is staged once in LDS with whole-row
// direct-to-LDS loads (row r's 16-byte chunk c in slot K/8 r + (c ^ (r & 15)),
// so the 16 rows of a fragment read fall on distinct bank groups) instead of
// every wave loading all of it from memory; the output tile reuses that LDS.
template <int N, int K, int TT, bool A_LDS>
__global__ __launch_bounds__(256, 2) void nt_gemm(GemmArgs g, int blocks_per_wg) {
  constexpr int ROWS = 16 * TT;     // tokens per block
  constexpr int NW = N / 4;         // output columns per wave
  constexpr int NT = NW / 16;       // column tiles per wave
  constexpr int KS = K / 32;        // k-steps
  constexpr int PITCH = 2 * N + 16; // bytes per row of the staged output tile
  constexpr int CPR = K / 8;        // 16-byte chunks per A row
  constexpr int OUT_BYTES = ROWS * PITCH;
  constexpr int A_BYTES = A_LDS ? ROWS * K * 2 : 0;
  static_assert(NT >= 1 && KS >= 1 && TT >= 1, "shape");
  static_assert(!A_LDS || CPR == 64, "A staging: one 1 KB row per wave load");
  __shared__ __attribute__((aligned(1024))) uint8_t tile[OUT_BYTES > A_BYTES ? OUT_BYTES : A_BYTES];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int i16 = lane & 15, gq = lane >> 4;
  // x: head, y: range of token blocks
  const size_t h = blockIdx.x;
  const int nblocks = (g.m + ROWS - 1) / ROWS;
  const int blk0 = blockIdx.y * blocks_per_wg;
  const int blk1 = min(nblocks, blk0 + blocks_per_wg);
  const uint16_t* A = g.a + h * g.a_head;
  const uint16_t* B = g.bt + h * g.b_head;
  uint16_t* C = g.c + h * g.c_head;

  // the wave's weight slice: rows NW w + 16 j + i16, features 32 ks + 8 gq .. + 7
  bf16x8 bc[KS][NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const uint16_t* brow = B + (size_t)(NW * w + 16 * j + i16) * g.b_row + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bc[ks][j] = *reinterpret_cast<const bf16x8*>(brow + 32 * ks);
  }

  for (int blk = blk0; blk < blk1; ++blk) {
    const int m0 = blk * ROWS;
    bf16x8 ac[A_LDS ? 1 : KS][A_LDS ? 1 : TT];
    if constexpr (A_LDS) {
      // rows past the last token repeat it (read, never used: their outputs are not stored)
      const int last = g.m - 1 - m0;
      MLA_LDS uint8_t* const dst = (MLA_LDS uint8_t*)tile;
#pragma unroll
      for (int i = 0; i < ROWS / 4; ++i) {  // wave load r: row r, lane l: chunk l ^ (r & 15)
        const int r = w + 4 * i;
        const uint16_t* src = A + (size_t)(m0 + (r < last ? r : last)) * g.a_row;
        lds_dma16(reinterpret_cast<const uint8_t*>(src), 16 * (lane ^ (r & 15)), dst + r * 1024);
      }
      wait_vmcnt<0>();
      __syncthreads();
    } else {
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        const int r = m0 + 16 * i + i16;
        const uint16_t* arow = A + (size_t)(r < g.m ? r : 0) * g.a_row + 8 * gq;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ac[ks][i] = r < g.m ? *reinterpret_cast<const bf16x8*>(arow + 32 * ks) : bf16x8{};
      }
    }
    auto a_frag = [&](int i, int ks) {  // rows 16 i + i16, features 32 ks + 8 gq .. + 7
      if constexpr (A_LDS) {
        const int r = 16 * i + i16;
        return *reinterpret_cast<const MLA_LDS bf16x8*>((const MLA_LDS uint8_t*)tile +
                                                         16 * (CPR * r + ((4 * ks + gq) ^ (r & 15))));
      } else {
        return ac[ks][i];
      }
    };
    f32x4 acc[NT][TT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < TT; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        const bf16x8 af = a_frag(i, ks);
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j][i] = mfma16x16x32(bc[ks][j], af, acc[j][i]);
      }

    if (A_LDS) __syncthreads();  // every wave is done with the staged A tile
    // lane holds C[16 i + i16][NW w + 16 j + 4 gq + e], e = 0..3
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        bf16x4 o;
        o[0] = (__bf16)acc[j][i][0]; o[1] = (__bf16)acc[j][i][1];
        o[2] = (__bf16)acc[j][i][2]; o[3] = (__bf16)acc[j][i][3];
        *reinterpret_cast<bf16x4*>(tile + (16 * i + i16) * PITCH + 2 * (NW * w + 16 * j + 4 * gq)) = o;
      }
    __syncthreads();
    // whole rows: N / 8 chunks of 16 bytes per token
    constexpr int OCPR = N / 8;
    static_assert(ROWS * OCPR % 256 == 0, "whole store rounds");
#pragma unroll
    for (int it = 0; it < ROWS * OCPR / 256; ++it) {
      const int c = threadIdx.x + 256 * it;
      const int r = c / OCPR, q = c - r * OCPR;
      if (m0 + r < g.m)
        *reinterpret_cast<u32x4*>(C + (size_t)(m0 + r) * g.c_row + 8 * q) =
            *reinterpret_cast<const u32x4*>(tile + r * PITCH + 16 * q);
    }
    // absorption: the rope columns of this block's tokens pass through unchanged
    if (g.rope_cols > 0) {
      const int chunks = g.rope_cols / 8;
      for (int c = threadIdx.x; c < ROWS * chunks; c += 256) {
        const int r = m0 + c / chunks;
        if (r >= g.m) continue;
        const int q = c - (c / chunks) * chunks;
        *reinterpret_cast<u32x4*>(g.rope_dst + h * g.rope_dst_head + (size_t)r * g.rope_dst_row + 8 * q) =
            *reinterpret_cast<const u32x4*>(g.rope_src + h * g.rope_src_head + (size_t)r * g.rope_src_row + 8 * q);
      }
    }
    __syncthreads();  // the staged tile is read out before the next block reuses it
  }
}

// Token blocks per workgroup: enough workgroups for two per compute unit
// (the kernel's occupancy), each taking a contiguous range of blocks.
template <int ROWS>
void gemm_grid(const GemmArgs& g, int heads, int cus, dim3& grid, int& per_wg) {
  const int nblocks = (g.m + ROWS - 1) / ROWS;
  const int target = 2 * (cus > 0 ? cus : 256);
  int ranges = (target + heads - 1) / heads;
  if (ranges > nblocks) ranges = nblocks;
  if (ranges < 1) ranges = 1;
  per_wg = (nblocks + ranges - 1) / ranges;
  grid = dim3(heads, (nblocks + per_wg - 1) / per_wg);
}

hipError_t launch_gemm(const GemmArgs& g, int heads, int cus, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  dim3 grid;
  int per_wg = 1;
  if (g.n == 512 && g.k == 128) {
    gemm_grid<32>(g, heads, cus, grid, per_wg);
    hipLaunchKernelGGL((nt_gemm<512, 128, 2, false>), grid, dim3(256), 0, stream, g, per_wg);
  } else if (g.n == 128 && g.k == 512) {
    gemm_grid<64>(g, heads, cus, grid, per_wg);
    hipLaunchKernelGGL((nt_gemm<128, 512, 4, true>), grid, dim3(256), 0, stream, g, per_wg);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
