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
// reason; W_UV[h] ([128][512]) already is.  A workgroup computes a 64 x 64
// tile of C with four waves of 32 x 32 (2 x 2 v_mfma_f32_16x16x32_bf16
// blocks), operands loaded straight from global memory (16 bytes per lane,
// the weights stay in L2 across token tiles) one k-step ahead.  The product
// is taken transposed (D = Bt A^T) so that each lane holds four consecutive
// output columns of one token and stores them as one 8-byte write.  fp32
// accumulation, bf16 output rounded to nearest even.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kGemmTile = 64;

__global__ __launch_bounds__(256) void nt_gemm(GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int i16 = lane & 15, gq = lane >> 4;
  const size_t h = blockIdx.z;
  const int m0 = blockIdx.x * kGemmTile + 32 * (w & 1);
  const int n0 = blockIdx.y * kGemmTile + 32 * (w >> 1);
  const uint16_t* A = g.a + h * g.a_head;
  const uint16_t* B = g.bt + h * g.b_head;

  const uint16_t* arow[2];
  bool aok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = m0 + 16 * i + i16;
    aok[i] = r < g.m;
    arow[i] = A + (size_t)(aok[i] ? r : 0) * g.a_row + 8 * gq;
  }
  const uint16_t* brow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) brow[j] = B + (size_t)(n0 + 16 * j + i16) * g.b_row + 8 * gq;

  auto load = [](const uint16_t* p, bool ok) {
    return ok ? *reinterpret_cast<const bf16x8*>(p) : bf16x8{};
  };
  bf16x8 ac[2], bc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) ac[i] = load(arow[i], aok[i]);
#pragma unroll
  for (int j = 0; j < 2; ++j) bc[j] = load(brow[j], true);
  f32x4 acc[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < g.k; k0 += 32) {
    bf16x8 an[2], bn[2];
    const bool more = k0 + 32 < g.k;
    if (more) {
#pragma unroll
      for (int i = 0; i < 2; ++i) an[i] = load(arow[i] + k0 + 32, aok[i]);
#pragma unroll
      for (int j = 0; j < 2; ++j) bn[j] = load(brow[j] + k0 + 32, true);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[j][i] = mfma16x16x32(bc[j], ac[i], acc[j][i]);
    if (more) {
#pragma unroll
      for (int i = 0; i < 2; ++i) ac[i] = an[i];
#pragma unroll
      for (int j = 0; j < 2; ++j) bc[j] = bn[j];
    }
  }

  // lane holds C[m0 + 16 i + i16][n0 + 16 j + 4 gq + e], e = 0..3
  uint16_t* C = g.c + h * g.c_head;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (!aok[i]) continue;
    uint16_t* crow = C + (size_t)(m0 + 16 * i + i16) * g.c_row + n0 + 4 * gq;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x4 o;
      o[0] = (__bf16)acc[j][i][0]; o[1] = (__bf16)acc[j][i][1];
      o[2] = (__bf16)acc[j][i][2]; o[3] = (__bf16)acc[j][i][3];
      *reinterpret_cast<bf16x4*>(crow + 16 * j) = o;
    }
  }

  // absorption: the rope columns of this tile's tokens pass through unchanged
  if (g.rope_cols > 0 && blockIdx.y == 0) {
    const int chunks = g.rope_cols / 8;
    for (int c = threadIdx.x; c < kGemmTile * chunks; c += 256) {
      const int r = blockIdx.x * kGemmTile + c / chunks;
      if (r >= g.m) continue;
      const int q = c - (c / chunks) * chunks;
      *reinterpret_cast<u32x4*>(g.rope_dst + h * g.rope_dst_head + (size_t)r * g.rope_dst_row + 8 * q) =
          *reinterpret_cast<const u32x4*>(g.rope_src + h * g.rope_src_head + (size_t)r * g.rope_src_row + 8 * q);
    }
  }
}

hipError_t launch_gemm(const GemmArgs& g, int heads, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  const dim3 grid((g.m + kGemmTile - 1) / kGemmTile, g.n / kGemmTile, heads);
  hipLaunchKernelGGL(nt_gemm, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace mla
