// Drives the library's host layer (mla_api.cpp, linked in) under AddressSanitizer
// and UndefinedBehaviorSanitizer, without a GPU: the kernel launchers and the two
// HIP runtime queries are replaced by stubs that check what the host layer hands
// them (every workspace region inside the caller's buffer and 256-byte aligned,
// the plan's sizes consistent) instead of launching anything.  Exits non-zero on
// a wrong status code or a failed check; the sanitizers abort on any memory
// error or undefined behaviour.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mla.h"
#include "mla_internal.h"

namespace {
int failures = 0;
const char* current = "";
const uint8_t* g_ws = nullptr;
size_t g_ws_bytes = 0;
alignas(256) uint8_t g_scratch[4096];  // stands in for the device scratch (never dereferenced)

void fail(const char* what) {
  std::fprintf(stderr, "FAIL [%s]: %s\n", current, what);
  ++failures;
}

void in_ws(const void* p, size_t bytes, const char* what) {
  const uint8_t* b = static_cast<const uint8_t*>(p);
  if (!p || (reinterpret_cast<uintptr_t>(p) & 255) || b < g_ws || b + bytes > g_ws + g_ws_bytes) fail(what);
}
}  // namespace

namespace mla {
hipError_t launch_decode(const DecodePlan& plan, const DecodeArgs& a, int kv_dtype, hipStream_t) {
  if (plan.grid < 1 || a.grid != plan.grid || a.rows < 1 || a.rows > MLA_MAX_DECODE_ROWS) fail("decode plan");
  if (!std::isfinite(a.scale_log2) || a.heads < 1 || a.batch < 1 || kv_dtype < 0 || kv_dtype > 2) fail("decode args");
  if (plan.grid > 1) {
    const size_t slots = (size_t)(plan.grid + a.batch) * a.rows;
    if (plan.workspace_bytes > g_ws_bytes) fail("decode workspace size");
    in_ws(a.part_o, slots * kDv * 2, "decode partial outputs");
    in_ws(a.part_lse, slots * 4, "decode partial lse");
    in_ws(a.cum_pages, (size_t)(a.batch + 1) * 4, "decode page prefix sums");
    const uint8_t* o_end = reinterpret_cast<const uint8_t*>(a.part_o) + slots * kDv * 2;
    const uint8_t* l_end = reinterpret_cast<const uint8_t*>(a.part_lse) + slots * 4;
    if (reinterpret_cast<const uint8_t*>(a.part_lse) < o_end || reinterpret_cast<const uint8_t*>(a.cum_pages) < l_end)
      fail("decode workspace regions overlap");
  }
  return hipSuccess;
}
hipError_t launch_prefill(const PrefillPlan& plan, const PrefillArgs& a, int, hipStream_t) {
  if (plan.grid < 1 || a.tok_per_tile < 1 || (long long)a.tok_per_tile * a.heads > 64 && a.tok_per_tile != 1)
    fail("prefill plan");
  in_ws(a.counter, 4, "prefill queue head");
  in_ws(a.order, (size_t)a.batch * 4, "prefill order");
  in_ws(a.tile_cum, (size_t)(a.batch + 1) * 4, "prefill tile counts");
  return hipSuccess;
}
hipError_t launch_append(const AppendArgs& a, int kv_dtype, hipStream_t) {
  if (a.total_new < 1 || (kv_dtype != 0) != (a.kv_scale != nullptr)) fail("append args");
  return hipSuccess;
}
hipError_t launch_gemm(const GemmArgs& g, int heads, int cus, hipStream_t) {
  if (g.m < 1 || heads < 1 || cus < 1 || !(g.n == 512 && g.k == 128) && !(g.n == 128 && g.k == 512)) fail("gemm args");
  return hipSuccess;
}
hipError_t noalloc_scratch(void** p) {
  *p = g_scratch;
  g_ws = g_scratch;
  g_ws_bytes = kNoAllocScratchBytes;
  return hipSuccess;
}
}  // namespace mla

extern "C" hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
extern "C" hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }

namespace {
void* const D = reinterpret_cast<void*>(0x10000);  // a device pointer the host layer never dereferences
const int32_t* const DI = reinterpret_cast<const int32_t*>(0x20000);

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL [%s]: %s: status %d, expected %d\n", current, what, got, want);
    ++failures;
  }
}

std::vector<uint8_t> ws_buf;
uint8_t* workspace(size_t bytes) {
  ws_buf.assign(bytes + 512, 0);
  uint8_t* p = ws_buf.data();
  p += (256 - (reinterpret_cast<uintptr_t>(p) & 255)) & 255;
  g_ws = p;
  g_ws_bytes = bytes;
  return p;
}
}  // namespace

int main() {
  setenv("MLA_NUM_CUS", "256", 1);
  const int kinds[3] = {MLA_KV_BF16, MLA_KV_INT8, MLA_KV_FP8};
  const int shapes[][4] = {{1, 16, 1, 256}, {4, 16, 4, 65536}, {16, 32, 2, 131072}, {8, 16, 4, 262144},
                           {3, 128, 1, 1000}, {2, 32, 4, 8192}, {37, 16, 2, 4096}, {1, 1, 1, 1}};
  for (int kind : kinds)
    for (auto& sh : shapes)
      for (int page : {64, 128, 1536}) {
        const int batch = sh[0], H = sh[1], q = sh[2], L = sh[3];
        current = "decode";
        size_t bytes = 0;
        expect(mla_splitkv_workspace_size(batch, H, q, batch * q, L, kind, &bytes), MLA_OK, "workspace size");
        uint8_t* ws = workspace(bytes);
        const int maxp = (L + page - 1) / page;
        const float* sc = kind ? reinterpret_cast<const float*>(D) : nullptr;
        expect(mla_decode(D, D, sc, kind, DI, maxp, DI, batch, q, H, page, L, 0.07f, D,
                          reinterpret_cast<float*>(D), bytes ? ws : nullptr, bytes, nullptr),
               MLA_OK, "valid decode");
        size_t plan_bytes = 0;
        int groups = 0;
        expect(mla_decode_plan(batch, H, q, L, kind, 256, &groups, &plan_bytes), MLA_OK, "decode plan");
        if (plan_bytes > bytes) fail("workspace size below the plan's");
        expect(mla_decode(D, D, sc, kind, DI, maxp, DI, batch, q, H, page, L, 0.07f, D,
                          reinterpret_cast<float*>(D), ws, plan_bytes ? plan_bytes - 1 : 0, nullptr),
               plan_bytes ? MLA_ERR_WORKSPACE : MLA_OK, "short workspace");
        std::vector<int32_t> cu(batch + 1);
        current = "decode_varlen";
        expect(mla_decode_varlen(D, cu.data(), D, sc, kind, DI, maxp, DI, batch, batch * q - 1 > 0 ? batch * q - 1 : 1,
                                 q, H, page, L, 0.07f, D, reinterpret_cast<float*>(D), bytes ? ws : nullptr, bytes,
                                 nullptr),
               MLA_OK, "valid varlen decode");
        current = "noalloc";
        expect(mla_decode_noalloc(D, D, sc, kind, DI, maxp, DI, batch, q, H, page, L, 0.07f, D,
                                  reinterpret_cast<float*>(D), nullptr),
               plan_bytes <= MLA_NOALLOC_SCRATCH_BYTES ? MLA_OK : MLA_ERR_SCRATCH, "noalloc decode");
        current = "prefill";
        const int T = batch * 3;
        const int mq = T < L ? (T < 5 ? T : 5) : L;
        expect(mla_splitkv_workspace_size(batch, H, mq, T, L, kind, &bytes), MLA_OK, "prefill workspace size");
        ws = workspace(bytes);
        expect(mla_prefill_varlen(D, DI, DI, D, sc, kind, DI, maxp, batch, T, mq, L, H, page, 0.07f, D,
                                  reinterpret_cast<float*>(D), ws, bytes, nullptr),
               T >= mq ? MLA_OK : MLA_ERR_INVALID, "valid prefill");
        current = "append";
        expect(mla_kv_append(D, DI, DI, D, kind ? reinterpret_cast<float*>(D) : nullptr, kind, DI, maxp, batch, T,
                             page, nullptr),
               MLA_OK, "valid append");
      }
  current = "invalid";
  expect(mla_decode(nullptr, D, nullptr, 0, DI, 1024, DI, 4, 4, 16, 64, 65536, 0.07f, D, reinterpret_cast<float*>(D),
                    nullptr, 0, nullptr),
         MLA_ERR_INVALID, "null query");
  expect(mla_decode(D, D, nullptr, 0, DI, 1024, DI, 4, 9, 16, 64, 65536, 0.07f, D, reinterpret_cast<float*>(D),
                    nullptr, 0, nullptr),
         MLA_ERR_UNSUPPORTED, "144 folded rows");
  expect(mla_decode(D, D, nullptr, 0, DI, 1024, DI, 4, 4, 16, 96, 65536, 0.07f, D, reinterpret_cast<float*>(D),
                    nullptr, 0, nullptr),
         MLA_ERR_UNSUPPORTED, "page size 96");
  expect(mla_decode(D, D, nullptr, 0, DI, 1024, DI, 4, 4, 16, 64, 65536, NAN, D, reinterpret_cast<float*>(D),
                    nullptr, 0, nullptr),
         MLA_ERR_INVALID, "NaN scale");
  expect(mla_decode(D, D, nullptr, 1, DI, 1024, DI, 4, 4, 16, 64, 65536, 0.07f, D, reinterpret_cast<float*>(D),
                    nullptr, 0, nullptr),
         MLA_ERR_INVALID, "int8 without scales");
  expect(mla_decode_noalloc(D, D, nullptr, 0, DI, 4096, DI, 4000, 4, 16, 64, 262144, 0.07f, D,
                            reinterpret_cast<float*>(D), nullptr),
         MLA_ERR_SCRATCH, "noalloc beyond its scratch");
  expect(mla_prefill_varlen(D, DI, DI, D, nullptr, 0, DI, 10, 2, 5, 6, 640, 16, 64, 0.07f, D,
                            reinterpret_cast<float*>(D), D, 4096, nullptr),
         MLA_ERR_INVALID, "max_q_len above total_q");
  current = "gemm";
  expect(mla_q_absorb(D, D, D, 8629, 16, nullptr), MLA_OK, "q_absorb");
  expect(mla_v_up(D, D, D, 8629, 16, nullptr), MLA_OK, "v_up");
  expect(mla_q_absorb(D, D, D, -1, 16, nullptr), MLA_ERR_INVALID, "q_absorb negative tokens");
  for (int s = -1; s < 8; ++s)
    if (!mla_status_string(s) || !*mla_status_string(s)) fail("status string");
  if (failures) {
    std::fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  std::puts("host driver ok");
  return 0;
}
