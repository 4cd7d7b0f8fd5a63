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
// spread over the 64 lanes (lanes 0..7 take a second chunk), requested before
// the row's request and page are looked up.  The INT8 and FP8 paths take the
// row's max magnitude with a wave reduction; each code is then the rounding
// of the correctly rounded fp32 quotient x / scale, as the definition reads
// (see row_quotients below).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kAppendWaves = 4;  // rows per workgroup

// E4M3 codes of four quotients (|q| <= 448 up to an fp32 rounding): gfx950's
// scaled fp32 -> FP8 conversion with scale 1, which rounds to the nearest
// OCP E4M3 value with ties to the even mantissa (subnormals included); two
// codes per conversion, src0 into the lower byte.
typedef short short2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3_codes4(float q0, float q1, float q2, float q3) {
  short2_cvt v = {0, 0};
  v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, q0, q1, 1.0f, false);
  v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, q2, q3, 1.0f, true);
  return __builtin_bit_cast(uint32_t, v);
}

// The correctly rounded quotients x / scale of one row's values, by the
// steps of the IEEE fp32 division (reciprocal estimate, one Newton step, the
// quotient and two residual corrections with fused multiply-adds) with the
// reciprocal refined once for the row's scale instead of once per value.
// For a scale in [2^-60, 2^60] and the row's |x| <= 448 scale those steps
// meet no overflow and no denormal that could matter (quotients below 2^-11
// give the code 0 either way), which is what the division's operand scaling
// and final fix-up guard against; any other scale (a wave-uniform choice)
// takes the division itself.  The quotient's sign is x's (scale > 0), which
// also keeps -0.
__device__ __forceinline__ void row_quotients(const float (&x)[2][8], float scale, float (&q)[2][8]) {
  const bool plain = __builtin_amdgcn_readfirstlane((int)(scale >= 0x1p-60f && scale <= 0x1p60f)) != 0;
  if (plain) {
    const float r0 = __builtin_amdgcn_rcpf(scale);
    const float r = fmaf(fmaf(-scale, r0, 1.0f), r0, r0);
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = x[k][e];
        float qv = xv * r;
        qv = fmaf(fmaf(-scale, qv, xv), r, qv);
        qv = fmaf(fmaf(-scale, qv, xv), r, qv);
        q[k][e] = copysignf(qv, xv);
      }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) q[k][e] = x[k][e] / scale;
  }
}

__global__ __launch_bounds__(kAppendWaves * 64) void kv_append(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  if (r >= a.total_new) return;
  // The row's chunks are requested first, so that their latency overlaps the
  // request lookup and the page-table read.
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kv_new + (size_t)r * kDqk);
  const bool two = lane < kRowChunks - 64;  // lanes holding a second chunk
  u32x4 u[2] = {*reinterpret_cast<const u32x4*>(src + 16 * lane), {0u, 0u, 0u, 0u}};
  if (two) u[1] = *reinterpret_cast<const u32x4*>(src + 16 * (lane + 64));
  // Request of row r: the largest b with cu[b] <= r.  cu does not decrease, so
  // the entries <= r are a prefix; each lane reads one entry (and its start
  // position) and a ballot finds the prefix's end, 64 requests per round trip.
  int b = 0, cu_b = 0, start_b = 0;
  for (int base = 0; base < a.batch; base += 64) {
    const int bb = base + lane;
    const int c = bb < a.batch ? a.cu[bb] : 0;
    const int sp = bb < a.batch ? a.start_pos[bb] : 0;
    const unsigned long long m = __ballot(bb < a.batch && c <= r);
    if (m == 0) break;  // never for the first 64 (cu[0] = 0 <= r)
    const int last = 63 - __clzll((long long)m);
    b = base + last;
    cu_b = __shfl(c, last);
    start_b = __shfl(sp, last);
    if (m != ~0ull) break;
  }
  const int t = start_b + (r - cu_b);
  if (t < 0 || t >= a.max_pages * kPage) return;  // outside the request's page table
  const size_t pos = (size_t)sub_page(a.page_table, (size_t)b * a.pt_stride, t >> 6, a.sub) * kPage + (t & (kPage - 1));

  if (a.kv_scale == nullptr) {  // bf16 cache: copy
    uint8_t* dst = a.kv + pos * kRowBytes;
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = u[0];
    if (two) *reinterpret_cast<u32x4*>(dst + 16 * (lane + 64)) = u[1];
    return;
  }

  // int8 cache: scale = max|x| / 127, code = clamp(rint(x / scale), -127, 127);
  // fp8 cache: scale = max|x| / 448, code = E4M3 nearest-even of x / scale
  const bool fp8 = a.code == kCodeFp8;
  float x[2][8];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[k][2 * e] = __uint_as_float(u[k][e] << 16);  // bf16 -> fp32 is exact
      x[k][2 * e + 1] = __uint_as_float(u[k][e] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(x[k][2 * e]), fabsf(x[k][2 * e + 1])));
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  float scale = fp8 ? amax / 448.0f : amax / 127.0f;
  if (scale == 0.f) scale = 1.0f;
  float q[2][8];
  row_quotients(x, scale, q);
  uint8_t* dst = a.kv + pos * kI8RowBytes;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (k == 1 && !two) break;
    u32x2 packed = {0u, 0u};
    if (fp8) {
      packed[0] = e4m3_codes4(q[k][0], q[k][1], q[k][2], q[k][3]);
      packed[1] = e4m3_codes4(q[k][4], q[k][5], q[k][6], q[k][7]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = fminf(fmaxf(__builtin_rintf(q[k][e]), -127.0f), 127.0f);
        packed[e >> 2] |= ((uint32_t)(int32_t)c & 0xffu) << (8 * (e & 3));
      }
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
