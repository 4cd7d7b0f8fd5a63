// KV append: write the rows of new tokens into their requests' pages, as a
// bf16 copy or as symmetric per-row INT8 or FP8 (E4M3) codes with an fp32
// scale.
//
// Sources (web pages on the TokenSpeed inference engine):
//   [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎", AICon 2026 talk
//          transcript, section "Kernel：让 MLA 真正跑满 GPU": attention runs
//          over a paged latent cache, one compressed row per token, and an
//          INT8 latent cache is one way to cut decode's bandwidth.
//   [GITREAD] "TokenSpeed 深度解析:把 LLM 推理压到"光速"意味着什么", section
//          "核心技术揭秘": FP8 KV-cache quantisation.  Read as OCP E4M3
//          (finite, largest magnitude 448), scale = max|x| / 448, values
//          rounded to the nearest E4M3 value with ties to even, saturating.
//
// One wave per new row; the row's 72 16-byte chunks (8 values each) are
// spread over the 64 lanes (lanes 0..7 take a second chunk).  The INT8 path
// takes the row's max magnitude with a wave reduction, then every lane
// quantises its values with IEEE fp32 division and round-half-even, exactly
// as the definition reads (no reciprocal, no fused shortcuts).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kAppendWaves = 4;  // rows per workgroup

// E4M3 code of a finite fp32 value: nearest E4M3 value, ties to the even
// mantissa, magnitudes above 448 saturating to 448.  For |q| >= 2^-6 (the
// normal binades) |q| * 2^-120 is an exact fp32 whose exponent field is the
// E4M3 exponent field and whose top 3 mantissa bits are the E4M3 mantissa;
// rounding its low 20 bits to nearest-even on the bit pattern (a carry moves
// into the exponent) gives the code's 7 magnitude bits.  Below 2^-6 the grid
// is 2^-9: rint(|q| * 512) (exact scaling) is the subnormal mantissa, and
// 8 lands on the smallest normal, whose code is also 8.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t u = __float_as_uint(a * 0x1p-120f);
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    mag = min(r >> 20, 0x7Eu);
  }
  return sign | mag;
}

__global__ __launch_bounds__(kAppendWaves * 64) void kv_append(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  if (r >= a.total_new) return;
  // request of row r: the largest b with cu[b] <= r
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int t = a.start_pos[b] + (r - a.cu[b]);
  if (t < 0 || t >= a.max_pages * kPage) return;  // outside the request's page table
  const size_t pos = (size_t)sub_page(a.page_table, (size_t)b * a.pt_stride, t >> 6, a.sub) * kPage + (t & (kPage - 1));
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kv_new + (size_t)r * kDqk);
  const bool two = lane < kRowChunks - 64;  // lanes holding a second chunk

  if (a.kv_scale == nullptr) {  // bf16 cache: copy
    uint8_t* dst = a.kv + pos * kRowBytes;
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = *reinterpret_cast<const u32x4*>(src + 16 * lane);
    if (two) *reinterpret_cast<u32x4*>(dst + 16 * (lane + 64)) = *reinterpret_cast<const u32x4*>(src + 16 * (lane + 64));
    return;
  }

  // int8 cache: scale = max|x| / 127, code = clamp(rint(x / scale), -127, 127);
  // fp8 cache: scale = max|x| / 448, code = E4M3 nearest-even of x / scale
  const bool fp8 = a.code == kCodeFp8;
  float x[2][8];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (k == 0 || two) u = *reinterpret_cast<const u32x4*>(src + 16 * (lane + 64 * k));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[k][2 * e] = __uint_as_float(u[e] << 16);           // bf16 -> fp32 is exact
      x[k][2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(x[k][2 * e]), fabsf(x[k][2 * e + 1])));
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  float scale = fp8 ? amax / 448.0f : amax / 127.0f;
  if (scale == 0.f) scale = 1.0f;
  uint8_t* dst = a.kv + pos * kI8RowBytes;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (k == 1 && !two) break;
    u32x2 packed = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qv = x[k][e] / scale;
      uint32_t code;
      if (fp8) {
        code = e4m3_code(qv);
      } else {
        const float c = fminf(fmaxf(__builtin_rintf(qv), -127.0f), 127.0f);
        code = (uint32_t)(int32_t)c & 0xffu;
      }
      packed[e >> 2] |= code << (8 * (e & 3));
    }
    *reinterpret_cast<u32x2*>(dst + 8 * (lane + 64 * k)) = packed;
  }
  if (lane == 0) a.kv_scale[pos] = scale;
}

hipError_t launch_append(const AppendArgs& args, int kv_dtype, hipStream_t stream) {
  (void)kv_dtype;  // the kernel keys on kv_scale (null for bf16) and args.code
  if (args.total_new <= 0) return hipSuccess;
  const int blocks = (args.total_new + kAppendWaves - 1) / kAppendWaves;
  hipLaunchKernelGGL(kv_append, dim3(blocks), dim3(kAppendWaves * 64), 0, stream, args);
  return hipGetLastError();
}

}  // namespace mla
