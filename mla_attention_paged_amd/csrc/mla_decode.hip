// MLA decode over a paged latent cache: split-KV phase one and the merge.
//
// Sources (web pages on the TokenSpeed inference engine):
//   [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎", AICon 2026 talk
//          transcript, section "Kernel：让 MLA 真正跑满 GPU": query x latent
//          key is the first product; decode is bandwidth-bound even at long
//          prefixes; query tokens are folded into the head axis; split-KV runs
//          as a partial phase and a reduction phase with a runtime-computed
//          split and workspace.
//   [NEWS] "英偉達力薦，小團隊兩個月開源一款「光速級」智能體推理引擎", section
//          "TokenSpeed 性能預覽": the decode kernel folds the query-sequence
//          axis into the head axis to fill the M tile of the first product.
//
// Decomposition.  Request b's q_len * heads query rows form one block
// (contiguous in memory, so the fold is free).  All requests' cache pages
// are laid end to end in one stream of P pages and phase one gives each of
// its G workgroups an equal, contiguous share floor(g*P/G) .. floor((g+1)*P/G)
// of that stream, whatever the per-request lengths are: a short request
// costs no idle workgroups and a long one is spread over many.  A
// workgroup that meets several requests in its share produces one partial
// (normalised output and log2-sum-exp of its rows) per request; workgroup g
// stores its partial for request b in slot g + b, which is unique because a
// share that reaches request b + 1 cannot reach back into request b - 1.
// The merge then reduces, per request, the partials of the workgroups whose
// shares intersect it.  Every cache byte is read from HBM once per call,
// and each page is read by one workgroup for all the request's rows.
#include <mutex>

#include "mla_device.h"
#include "mla_internal.h"
#include "mla_ws.h"

namespace mla {

constexpr int kWin = 128;  // pages per window of the per-workgroup page list

__device__ __forceinline__ int clamp_len(int L, int max_pages) {
  L = L < 0 ? 0 : L;
  const int cap = max_pages * kPage;
  return L > cap ? cap : L;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d);
    if (lane >= d) v += y;
  }
  return v;
}

// First workgroup whose share contains global page p (shares are
// floor(g*P/G) .. floor((g+1)*P/G); the largest g with start <= p).
__device__ __forceinline__ int owner_group(long long p, long long P, int G) {
  return (int)(((p + 1) * G - 1) / P);
}

// Write the rows of one finished (request, share) pair: the final output
// (rows of the request whose first query token is tok0) when phase one is
// the only phase, else the partial in slot `slot`.  Wave
// half h writes value columns 256h .. 256h + 255; half 0 writes the LSE.
// Partial outputs are normalised (o / sum, a weighted mean of value rows)
// and stored in bf16 like the final output, halving the workspace traffic;
// their log2-sum-exp stays fp32.
__device__ __forceinline__ void flush_rows(const DecodeArgs& a, const RowState& st, int tok0, int slot,
                                           int row, bool row_ok, int half, int lane) {
  float inv, lse2;
  finish_row(st, inv, lse2);
  if (!row_ok) return;
  const int g = lane >> 4;
  const int col0 = (kDv / 2) * half + 4 * g;
  const bool final_out = a.grid == 1;
  uint16_t* dst = (final_out ? a.out + ((size_t)tok0 * a.heads + row) * kDv
                             : a.part_o + ((size_t)slot * a.rows + row) * kDv) + col0;
#pragma unroll
  for (int ct = 0; ct < kOHalf; ++ct) {
    const f32x4 v = st.o[ct] * inv;
    bf16x4 h;
    h[0] = (__bf16)v[0]; h[1] = (__bf16)v[1]; h[2] = (__bf16)v[2]; h[3] = (__bf16)v[3];
    *reinterpret_cast<bf16x4*>(dst + 16 * ct) = h;
  }
  if (g == 0 && half == 0) {
    if (final_out)
      a.lse[(size_t)tok0 * a.heads + row] = lse2 * kLn2;
    else
      a.part_lse[(size_t)slot * a.rows + row] = lse2;
  }
}

// The last flush of a workgroup, through LDS: every wave's normalised bf16
// rows go, row-major with a 1040-byte pitch, into `buf` (the idle ring),
// and then each wave stores whole 1 KB rows of the block (rows 8w .. 8w+7
// that the request has: nrows of them), so every store instruction fills
// eight 128-byte lines instead of touching sixteen lines 32 bytes at a time.
// All waves of the workgroup call it (barriers inside).
constexpr int kFlushPitch = kDv * 2 + 16;

__device__ __forceinline__ void flush_rows_lds(const DecodeArgs& a, const RowState& st, int tok0, int slot,
                                               int nrows, int row, bool row_ok, bool wave_rows, int half, int w,
                                               int lane, MLA_LDS uint8_t* buf) {
  lds_barrier();  // every wave is done reading the ring
  if (wave_rows) {
    float inv, lse2;
    finish_row(st, inv, lse2);
    const int g = lane >> 4;
    MLA_LDS uint8_t* dst = buf + (16 * (w & 3) + (lane & 15)) * kFlushPitch + 2 * ((kDv / 2) * half + 4 * g);
#pragma unroll
    for (int ct = 0; ct < kOHalf; ++ct) {
      const f32x4 v = st.o[ct] * inv;
      bf16x4 h;
      h[0] = (__bf16)v[0]; h[1] = (__bf16)v[1]; h[2] = (__bf16)v[2]; h[3] = (__bf16)v[3];
      *reinterpret_cast<MLA_LDS bf16x4*>(dst + 32 * ct) = h;
    }
    if (row_ok && g == 0 && half == 0) {
      if (a.grid == 1)
        a.lse[(size_t)tok0 * a.heads + row] = lse2 * kLn2;
      else
        a.part_lse[(size_t)slot * a.rows + row] = lse2;
    }
  }
  lds_write_barrier();
  const int r0 = kBlockRows * blockIdx.y;
  uint16_t* const base = a.grid == 1 ? a.out + ((size_t)tok0 * a.heads + r0) * kDv
                                     : a.part_o + ((size_t)slot * a.rows + r0) * kDv;
#pragma unroll
  for (int k = 0; k < kBlockRows / kWaves; ++k) {
    const int rr = (kBlockRows / kWaves) * w + k;
    if (rr < nrows) {
      const bf16x8 x = *reinterpret_cast<const MLA_LDS bf16x8*>(buf + rr * kFlushPitch + 16 * lane);
      *reinterpret_cast<bf16x8*>(base + (size_t)rr * kDv + 8 * lane) = x;
    }
  }
}

// Clamped request lengths, cached in LDS for the first kLenCache requests
// (the tile-list walks read them repeatedly; the cache keeps those reads
// off the global-memory latency chain in front of the first tile).
constexpr int kLenCache = 512;

struct Lens {
  const DecodeArgs& a;
  const int* cache;
  __device__ int operator()(int b) const {
    return b < kLenCache ? cache[b] : clamp_len(a.seq_lens[b], a.max_pages);
  }
};

// Query tokens of request b: its first token and its count (uniform q_len,
// or the per-request offsets, cached in LDS like the lengths).
struct ReqQ {
  int tok0, n;
};

__device__ __forceinline__ ReqQ req_q(const DecodeArgs& a, const int* s_tok, int b) {
  if (!a.cu_q) return {b * a.q_len, a.q_len};
  if (b < kLenCache) return {s_tok[b], s_tok[b + 1] - s_tok[b]};
  const int t0 = a.cu_q[b];
  return {t0, a.cu_q[b + 1] - t0};
}

// A share of the page stream: pages lo .. hi - 1, starting at page j0 of
// request b0 (b0 = batch when the share is empty).
struct Share {
  int lo, hi, b0, j0;
};

// Wave 0 of workgroup g locates its share floor(g*P/G) .. floor((g+1)*P/G)
// of the page stream and the (request, page) where it starts (returned, and
// stored in s_info[0..3] for the other waves), and fills the length cache
// (and, for per-request query counts, the token-offset cache, entries 0 ..
// min(batch, kLenCache)); workgroup (0, 0) also records the page prefix sums
// for the merge.
__device__ __forceinline__ Share locate_share(const DecodeArgs& a, int g, int lane, int* s_info, int* s_len,
                                              int* s_tok) {
  if (a.cu_q)
    for (int b = lane; b <= a.batch && b <= kLenCache; b += 64) s_tok[b] = a.cu_q[b];
  const int G = a.grid;
  long long P = 0;
  const bool write_cum = g == 0 && blockIdx.y == 0 && G > 1;
  for (int base = 0; base < a.batch; base += 64) {
    const int b = base + lane;
    const int L = b < a.batch ? clamp_len(a.seq_lens[b], a.max_pages) : 0;
    if (b < a.batch && b < kLenCache) s_len[b] = L;
    const int np = (L + kPage - 1) / kPage;
    const int incl = wave_incl_scan(np, lane);
    if (write_cum && b < a.batch) a.cum_pages[b] = (int)(P + incl - np);
    P += __shfl(incl, 63);
  }
  if (write_cum && lane == 0) a.cum_pages[a.batch] = (int)P;
  const Lens lens{a, s_len};  // lane b reads back the entry it wrote
  const long long lo = P * g / G, hi = P * (g + 1) / G;
  int b0 = a.batch, j0 = 0;
  if (lo < hi) {
    long long run = 0;
    for (int base = 0; base < a.batch; base += 64) {
      const int b = base + lane;
      const int np = b < a.batch ? (lens(b) + kPage - 1) / kPage : 0;
      const int incl = wave_incl_scan(np, lane);
      const long long before = run + incl - np;
      const bool hit = np > 0 && before <= lo && lo < before + np;
      const unsigned long long mask = __ballot(hit);
      if (mask) {
        const int src = __ffsll((long long)mask) - 1;
        b0 = base + src;
        j0 = (int)(lo - (run + __shfl(incl - np, src)));
        break;
      }
      run += __shfl(incl, 63);
    }
  }
  if (lane == 0) {
    s_info[0] = (int)lo;
    s_info[1] = (int)hi;
    s_info[2] = b0;
    s_info[3] = j0;
  }
  return {(int)lo, (int)hi, b0, j0};
}

// Orders this wave's earlier LDS writes before its later LDS reads of the
// same locations by other lanes.  The hardware performs a wave's LDS
// accesses in order; without a fence the compiler may still move a read of
// another lane's entry above the write (no barrier separates them).
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// A window's tile list (one wave builds it): the valid tiles (half pages
// holding at least one of their request's rows) of the n pages of the stream
// from request cb, page cj on, in stream order.  Tile t: page s_pid[t],
// request s_req[t] >> 1, half s_req[t] & 1, s_rem[t] = the request's rows
// from the tile's first row (> 0).  The tile count goes to *s_count.
__device__ __forceinline__ void window_tiles(const DecodeArgs& a, const Lens& lens, int n, int cb, int cj,
                                             int* s_pid, int* s_req, int* s_rem, int* s_count, int lane) {
  {
    int base = 0;
    for (int k0 = 0; k0 < n; k0 += 64) {
      const int k = k0 + lane;
      int nt = 0, b = cb, off = cj + k, Lc = 0;
      if (k < n) {
        for (;;) {
          Lc = lens(b);
          const int np = (Lc + kPage - 1) / kPage;
          if (off < np || b + 1 >= a.batch) break;
          off -= np;
          ++b;
        }
        off = min(off, a.max_pages - 1);  // never past the table, whatever the lengths say
        nt = Lc - kPage * off > kTileRows ? 2 : 1;
      }
      const int incl = wave_incl_scan(nt, lane);
      if (k < n) {
        const int t = base + incl - nt;
        const int pid = sub_page(a.page_table, (size_t)b * a.pt_stride, off, a.sub);
        const int rem = Lc - kPage * off;
        s_pid[t] = pid;
        s_req[t] = 2 * b;
        s_rem[t] = rem;
        if (nt == 2) {
          s_pid[t + 1] = pid;
          s_req[t + 1] = 2 * b + 1;
          s_rem[t + 1] = rem - kTileRows;
        }
      }
      base += __shfl(incl, 63);
    }
    if (lane == 0) *s_count = base;
  }
}

// Move the cursor (request cb, page cj) past n pages of the stream (every
// thread, with the same result).
__device__ __forceinline__ void advance_cursor(const DecodeArgs& a, const Lens& lens, int n, int& cb, int& cj) {
  int b = cb, off = cj + n;
  for (;;) {
    const int np = (lens(b) + kPage - 1) / kPage;
    if (off < np || b + 1 >= a.batch) break;
    off -= np;
    ++b;
  }
  cb = b;
  cj = off;
}

// Phase one for a bf16 cache, software-pipelined across tiles.  The
// window's tiles are processed in segments of one request each.  Step t of
// a segment waits for tile t (the only load in flight), passes one
// workgroup barrier, starts tile t + 1 into the third ring stage, and then
// computes the scores of tile t interleaved with the softmax of tile t - 1,
// hands its half of the scores to the partner wave through a
// double-buffered exchange, and accumulates the values of tile t - 1.  The
// first step of a segment only computes scores; after its last step one
// more barrier lets the partners finish the segment's last tile.  Query
// fragments are loaded and partials written only between segments.
__global__ __launch_bounds__(kWaves * 64, 2) void decode_phase1_pipe(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring_raw[kPStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) f32x4 xchg_raw[2 * kWaves * 64];
  MLA_LDS uint8_t* const ring = (MLA_LDS uint8_t*)ring_raw;
  MLA_LDS f32x4* const xchg = (MLA_LDS f32x4*)xchg_raw;
  __shared__ int s_pid[2 * kWin], s_req[2 * kWin], s_rem[2 * kWin];
  __shared__ int s_info[5];
  __shared__ int s_len[kLenCache];
  __shared__ int s_tok[kLenCache + 1];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = blockIdx.x;
  auto stage = [&](int t) { return ring + (t % kPStages) * kStageBytes; };

  // Guessed start.  The share, its first tile and its query block wait on
  // two dependent loads (the lengths, then the page table).  If every
  // request held max_seq_len rows, share g would start at page jg of request
  // bg.  While wave 0 locates the share, waves 1-7 load bg's length and page
  // jg's table entry, stage bg's query block while those loads are out, and
  // then request page jg's first tile if the page exists.  When the located
  // share starts at page jg of request bg (so the page exists), both are
  // already on their way; otherwise the waves drain them and the normal start
  // follows.  The test of the query pointer (never null here) makes it load
  // with the first arguments, before the guessed loads go out: a later first
  // use would wait for every outstanding scalar load, theirs included.
  int bg = -1, jg = 0;
  if (a.guess_pages > 0 && a.q != nullptr) {
    const long long Pg = (long long)a.batch * a.guess_pages;
    const long long lo = Pg * g / a.grid;
    if (lo < Pg * (g + 1) / a.grid) {
      bg = (int)(lo / a.guess_pages);
      jg = (int)(lo - (long long)bg * a.guess_pages);
    }
  }
  if (w == 0) {
    const Share sh = locate_share(a, g, lane, s_info, s_len, s_tok);
    // the first window's tile list, while waves 1-7 issue their loads (its
    // length lookups read the cache entries other lanes just wrote)
    wave_lds_fence();
    if (sh.lo < sh.hi)
      window_tiles(a, Lens{a, s_len}, min(kWin, sh.hi - sh.lo), sh.b0, sh.j0, s_pid, s_req, s_rem, &s_info[4], lane);
  } else if (bg >= 0) {
    const int len_g = clamp_len(a.seq_lens[bg], a.max_pages);
    const int pid_g = sub_page(a.page_table, (size_t)bg * a.pt_stride, jg, a.sub);
    const int nrows = min(a.rows - kBlockRows * (int)blockIdx.y, kBlockRows);
    if (nrows > 0)
      stage_q(a.q + ((size_t)bg * a.rows + kBlockRows * blockIdx.y) * kDqk, nrows, stage(1), w - 1, kWaves - 1,
              lane);
    if (jg < (len_g + kPage - 1) / kPage)
      stage_tile<kWaves - 1>(a.kv + (size_t)pid_g * kPageBytes, 0, len_g - kPage * jg, stage(0), w - 1, lane);
  }
  __syncthreads();
  const Lens lens{a, s_len};
  const int seg_lo = s_info[0], seg_hi = s_info[1];
  const bool guessed = bg >= 0 && s_info[2] == bg && s_info[3] == jg && seg_lo < seg_hi;
  if (!guessed) wait_vmcnt<0>();  // no guessed load may land after the stages are reused
  if (seg_lo >= seg_hi) return;   // empty share (more workgroups than pages)
  int cb = s_info[2], cj = s_info[3];

  const int half = w >> 2;
  const int row = kBlockRows * blockIdx.y + 16 * (w & 3) + (lane & 15);
  const bool wave_rows = kBlockRows * blockIdx.y + 16 * (w & 3) < a.rows;
  // the current request's query rows: this lane's row exists when
  // row < n * heads, and its token (row / heads) sees rows t <= L - late
  bool row_ok = false;
  int late = 0, tok0 = 0;
  auto set_req = [&](int b) {
    const ReqQ r = req_q(a, s_tok, b);
    row_ok = row < r.n * a.heads;
    late = r.n - (row_ok ? row / a.heads : 0);
    tok0 = r.tok0;
  };
  MLA_LDS f32x4* const xmine = xchg + 64 * w + lane;
  MLA_LDS f32x4* const xpart = xchg + 64 * (w ^ 4) + lane;

  RowState st;
  bf16x8 qf[kQFrags];
  int cur_b = -1;
  // The first request's query block streams into ring stages 1-2 (free
  // until the first step issues tile 1) in whole-line direct-to-LDS loads,
  // issued by waves 1-7 while wave 0 fills the tile list; the first step's
  // wait covers them and the first step moves the block into registers.
  // (Per-lane fragment loads from HBM touch every line twice, half a line at
  // a time, and took several microseconds here; the same loads issued after
  // the first tile's delay that tile by about 2 us.)
  const int q_b = cb;  // request whose query block is staged
  bool q_staged = true;
  if (w > 0 && !guessed) {
    const ReqQ r = req_q(a, s_tok, q_b);
    const int nrows = min(r.n * a.heads - kBlockRows * (int)blockIdx.y, kBlockRows);
    if (nrows > 0)
      stage_q(a.q + ((size_t)r.tok0 * a.heads + kBlockRows * blockIdx.y) * kDqk, nrows, stage(1), w - 1,
              kWaves - 1, lane);
  }

  for (int wlo = seg_lo; wlo < seg_hi; wlo += kWin) {
    const int n = min(kWin, seg_hi - wlo);
    if (wlo != seg_lo) {  // the first window's list was built before the first barrier
      __syncthreads();    // the previous window's list and stages are no longer read
      if (w == 0) window_tiles(a, lens, n, cb, cj, s_pid, s_req, s_rem, &s_info[4], lane);
      __syncthreads();
    }
    advance_cursor(a, lens, n, cb, cj);
    const int N = s_info[4];
    auto issue = [&](int t) {
      stage_tile<kWaves>(a.kv + (size_t)s_pid[t] * kPageBytes, s_req[t] & 1, s_rem[t] + kTileRows * (s_req[t] & 1),
                         stage(t), w, lane);
    };
    if (!guessed || wlo != seg_lo) issue(0);
    for (int t0 = 0; t0 < N;) {
      const int b = s_req[t0] >> 1;
      // the segment ends at the first later tile of another request: a
      // wave-wide compare of 64 list entries at a time (one entry per step
      // would put an LDS round trip per tile in front of the first tile)
      int t1 = N;
      for (int base = t0 + 1; base < N; base += 64) {
        const unsigned long long m = __ballot(base + lane < N && (s_req[base + lane] >> 1) != b);
        if (m) {
          t1 = base + __ffsll((long long)m) - 1;
          break;
        }
      }
      if (wave_rows && b != cur_b) {
        if (cur_b >= 0) flush_rows(a, st, tok0, g + cur_b, row, row_ok, half, lane);
        set_req(b);
        if (b != q_b) load_q(row_ok ? a.q + ((size_t)tok0 * a.heads + row) * kDqk : nullptr, lane, qf);
        reset_state(st);
      }
      cur_b = b;
      // first step: scores only
      wait_vmcnt<0>();
      lds_write_barrier();
      if (q_staged) {  // the first request's block, then free stages 1-2 for the ring
        if (wave_rows) read_q(stage(1), w & 3, lane, row_ok, qf);
        lds_write_barrier();
        q_staged = false;
      }
      if (t0 + 1 < N) issue(t0 + 1);
      f32x4 s_prev = {0.f, 0.f, 0.f, 0.f};
      if (wave_rows) {
        s_prev = tile_scores(stage(t0), qf, lane, half);
        xmine[(t0 & 1) * kWaves * 64] = s_prev;
      }
      int prev_lim = s_rem[t0] - late;
      for (int t = t0 + 1; t < t1; ++t) {
        wait_vmcnt<0>();
        lds_write_barrier();
        if (t + 1 < N) issue(t + 1);
        const int lim = s_rem[t] - late;
        if (wave_rows) {
          const f32x4 other = xpart[((t - 1) & 1) * kWaves * 64];
          const f32x4 lo = half == 0 ? s_prev : other;
          const f32x4 hi = half == 0 ? other : s_prev;
          s_prev = tile_step(stage(t), stage(t - 1), qf, lo, hi, prev_lim, a.scale_log2, lane, half, st);
          xmine[(t & 1) * kWaves * 64] = s_prev;
        }
        prev_lim = lim;
      }
      // last tile of the segment
      lds_write_barrier();
      if (wave_rows) {
        const f32x4 other = xpart[((t1 - 1) & 1) * kWaves * 64];
        const f32x4 lo = half == 0 ? s_prev : other;
        const f32x4 hi = half == 0 ? other : s_prev;
        float alpha;
        const bf16x8 pb = tile_softmax(lo, hi, prev_lim, a.scale_log2, lane, st, alpha);
        rescale_o(st, alpha);
        tile_values(stage(t1 - 1), pb, lane, half, st);
      }
      t0 = t1;
    }
  }
  if (cur_b >= 0) {
    const ReqQ r = req_q(a, s_tok, cur_b);
    const int nrows = min(r.n * a.heads - kBlockRows * (int)blockIdx.y, kBlockRows);
    flush_rows_lds(a, st, r.tok0, g + cur_b, nrows, row, row_ok, wave_rows, half, w, lane, ring);
  }
}

// Phase one for an INT8 or FP8 cache (CODE) on the wave-specialised core of
// the prefill kernels (mla_ws.h): score waves and value waves, the codes
// loaded into the value waves' registers and widened to bf16 while the score
// waves compute, the V fragments read behind the value MFMAs.  Workgroup g
// walks its share of the page stream one request segment at a time: the
// request's folded rows (row block blockIdx.y) against the share's pages of
// that request, written as the partial of slot g + b (or, with a single
// workgroup, as the final output).  The merge is the bf16 decode's.
template <int CODE>
__global__ __launch_bounds__(kWaves * 64, 2) void decode_ws_codes(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t cvt_raw[3 * kStageBytes];
  __shared__ __attribute__((aligned(16))) float tsc_raw[3 * kTileRows];
  __shared__ __attribute__((aligned(16))) float mx_raw[4 * 2 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t pb_raw[2 * 2 * 64 * 16];
  __shared__ __attribute__((aligned(16))) float al_raw[2 * 2 * 64];
  __shared__ int s_pid[kPWin];
  __shared__ int s_info[5];
  __shared__ int s_len[kLenCache];
  __shared__ int s_tok[kLenCache + 1];
  const WsCodesLds L{(MLA_LDS uint8_t*)cvt_raw, (MLA_LDS float*)tsc_raw, (MLA_LDS float*)mx_raw,
                     (MLA_LDS uint8_t*)pb_raw, (MLA_LDS float*)al_raw, s_pid};
  const int lane = threadIdx.x & 63;
  const int w = wave_uniform(threadIdx.x >> 6);
  const int g = blockIdx.x;
  if (w == 0) locate_share(a, g, lane, s_info, s_len, s_tok);
  __syncthreads();
  const Lens lens{a, s_len};
  const WsArgs wa{a.kv, a.kv_scale, a.page_table, a.pt_stride, a.sub, a.scale_log2};
  int left = wave_uniform(s_info[1] - s_info[0]);  // pages of the share
  int j = wave_uniform(s_info[3]);                 // first page of the share in its first request
  for (int b = wave_uniform(s_info[2]); left > 0 && b < a.batch; ++b, j = 0) {
    const int L_b = wave_uniform(lens(b));
    const int take = min(left, (L_b + kPage - 1) / kPage - j);
    if (take <= 0) continue;
    left -= take;
    const ReqQ r = req_q(a, s_tok, b);
    WsBlock k;
    k.q = a.q + (size_t)r.tok0 * a.heads * kDqk;
    if (a.grid == 1) {
      k.out = a.out + (size_t)r.tok0 * a.heads * kDv;
      k.lse = a.lse + (size_t)r.tok0 * a.heads;
      k.lse_mul = kLn2;
    } else {
      k.out = a.part_o + (size_t)(g + b) * a.rows * kDv;
      k.lse = a.part_lse + (size_t)(g + b) * a.rows;
      k.lse_mul = 1.f;  // partial log-sum-exp in log2 units, as the merge reads it
    }
    k.r0 = kBlockRows * blockIdx.y;
    k.nrows = r.n * a.heads;
    k.vis0 = L_b - r.n;
    k.heads = a.heads;
    k.b = b;
    k.p_lo = j;
    k.p_hi = j + take;
    k.kv_end = L_b;
    if (k.r0 >= k.nrows) continue;  // this row block has no rows of the request
    __syncthreads();                // the previous segment is done with the LDS
    const WsBlock ku = wave_uniform(k);
    constexpr int kAhead = CODE == kCodeInt8 ? kKAheadDecodeInt8 : kKAheadC;
    if (w < 4)
      ws_codes_range<true, CODE, kAhead>(wa, ku, L, w, lane);
    else
      ws_codes_range<false, CODE, kAhead>(wa, ku, L, w, lane);
  }
}

// Phase two: per (request, row), reduce the partials of the workgroups
// whose shares intersect the request: lse = log2-sum-exp of the partial
// lses, out = sum_s 2^(lse_s - lse) o_s.  One workgroup per (row, quarter of
// the value columns); thread (group j, quad c) accumulates shares j, j + 8,
// ... for columns 4c .. 4c+3 of the quarter, eight partial loads in flight
// at once, and the eight groups are combined through LDS.  Two dependent
// memory round trips: the page offsets (with the query offsets), then each
// thread's share lse (thread i: share i) together with its group's first
// eight partials; the block max m of the lses and the weights 2^(lse_s - m)
// (0 for empty shares) then come from registers and LDS.  Requests with more
// than 64 shares load further batches of partials; more than 256 (a grid
// beyond 256 workgroups) reload the lses of each later chunk of 256.  Empty
// shares read the first share's (written, finite) slot with weight 0, so
// bytes of the workspace that phase one did not write never enter the sums.
constexpr int kMergeGroups = 8;
constexpr int kMergeChunk = 256;  // share weights held in LDS at a time

__device__ __forceinline__ bool share_empty(long long P, int G, int gg) {
  return P * gg / G >= P * (gg + 1) / G;
}

__global__ __launch_bounds__(256) void decode_merge(DecodeArgs a) {
  __shared__ float s_wgt[kMergeChunk];
  __shared__ float s_red[4];
  __shared__ f32x4 s_acc[kMergeGroups][32];
  __shared__ float s_ws[kMergeGroups];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int R = blockIdx.x;
  const int quarter = blockIdx.y;
  const int b = R / a.rows, row = R - b * a.rows;
  // round trip 1: page offsets and query offsets, loaded together
  const long long P = a.cum_pages[a.batch];
  const long long p0 = a.cum_pages[b], p1 = a.cum_pages[b + 1];
  int tok0 = b * a.q_len, nq = a.q_len;
  if (a.cu_q) {
    tok0 = a.cu_q[b];
    nq = a.cu_q[b + 1] - tok0;
  }
  if (row >= nq * a.heads) return;  // a row the request does not have
  if (p1 <= p0) return;
  const size_t orow = (size_t)tok0 * a.heads + row;  // output row
  const int G = a.grid;
  const int g0 = owner_group(p0, P, G), g1 = owner_group(p1 - 1, P, G);
  const int ns = g1 - g0 + 1;
  const float* lse_col = a.part_lse + (size_t)(g0 + b) * a.rows + row;  // share i: lse_col[i * rows]

  const int grp = tid >> 5, quad = tid & 31;
  const int col = quarter * (kDv / 4) + 4 * quad;
  const uint16_t* o_col = a.part_o + ((size_t)(g0 + b) * a.rows + row) * kDv + col;  // share i: + i * rows * 512
  const size_t share_stride = (size_t)a.rows * kDv;
  // shares can be empty only when there are fewer pages than workgroups
  const bool sparse = P < G;
  auto has_share = [&](int i) { return i < ns && (!sparse || !share_empty(P, G, g0 + i)); };
  auto share_lse = [&](int i) { return has_share(i) ? lse_col[(size_t)i * a.rows] : -INFINITY; };
  // the partials of shares k, k + 8, ..., k + 56 (the first share's slot where a share is missing or empty)
  auto load_batch = [&](int k, f32x4 (&v)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = k + u * kMergeGroups;
      const int src = has_share(i) ? i : 0;
      const bf16x4 x = *reinterpret_cast<const bf16x4*>(o_col + (size_t)src * share_stride);
      v[u] = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    }
  };

  // round trip 2: this thread's share lses and its group's first batch of partials
  const float l_own = share_lse(tid);
  f32x4 v[8];
  load_batch(grp, v);
  float m = l_own;
  for (int i = tid + kMergeChunk; i < ns; i += kMergeChunk) m = fmaxf(m, share_lse(i));
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
  if (lane == 0) s_red[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float m_use = m == -INFINITY ? 0.f : m;
  s_wgt[tid] = fast_exp2(l_own - m_use);  // 0 past the shares and for empty ones

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  bool loaded = true;  // v holds shares grp, grp + 8, ... of the first chunk
  for (int c0 = 0; c0 < ns; c0 += kMergeChunk) {
    const int nc = min(kMergeChunk, ns - c0);
    if (c0 > 0) {
      __syncthreads();  // the previous chunk's weights are no longer read
      s_wgt[tid] = fast_exp2(share_lse(c0 + tid) - m_use);
    }
    __syncthreads();
    for (int k0 = grp; k0 < nc; k0 += 8 * kMergeGroups) {
      if (!loaded) load_batch(c0 + k0, v);
      loaded = false;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wt = s_wgt[k0 + u * kMergeGroups];  // k0 + 8u < 256: 0 past the chunk's shares
        acc += v[u] * wt;
        wsum += wt;
      }
    }
  }
  s_acc[grp][quad] = acc;
  if (quad == 0) s_ws[grp] = wsum;
  __syncthreads();
  if (tid < 32) {
    f32x4 o = s_acc[0][tid];
    float tot = s_ws[0];
#pragma unroll
    for (int j = 1; j < kMergeGroups; ++j) {
      o += s_acc[j][tid];
      tot += s_ws[j];
    }
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
    bf16x4 h;
    h[0] = (__bf16)(o[0] * inv); h[1] = (__bf16)(o[1] * inv);
    h[2] = (__bf16)(o[2] * inv); h[3] = (__bf16)(o[3] * inv);
    *reinterpret_cast<bf16x4*>(a.out + orow * kDv + col) = h;
    if (quarter == 0 && tid == 0) a.lse[orow] = tot > 0.f ? (m_use + fast_log2(tot)) * kLn2 : -INFINITY;
  }
}

// The merge for batches whose requests each meet few shares: one workgroup
// per (request, block of kMergeRows rows, quarter of the value columns), an
// eighth as many workgroups as decode_merge.  Half-wave j merges row
// kMergeRows rb + j on its own, in share order with a running maximum: the
// lses and partials of kMergeDepth shares are requested together, then
// folded in one after another (a larger lse rescales the sum so far).  One
// dependent round trip per kMergeDepth shares and no barrier.  decode_merge,
// whose threads split the shares of one row, stays faster when each request
// meets many shares (4 requests of 64 rows, 64 workgroups each: 77-79 us
// per decode call with this kernel against 70-71 us), so launch_decode takes
// this kernel only for plans with at most
// kMergeRowsShares workgroups per request on average.  Empty shares (lse
// -inf) get weight 0 and read the first share's slot, as in decode_merge.
constexpr int kMergeRows = 8;
constexpr int kMergeDepth = 8;
constexpr int kMergeRowsShares = 40;

__global__ __launch_bounds__(256) void decode_merge_rows(DecodeArgs a) {
  const int grp = threadIdx.x >> 5, quad = threadIdx.x & 31;
  const int row_blocks = (a.rows + kMergeRows - 1) / kMergeRows;
  const int b = blockIdx.x / row_blocks;
  const int row = kMergeRows * (blockIdx.x - b * row_blocks) + grp;
  const int quarter = blockIdx.y;
  const long long P = a.cum_pages[a.batch];
  const long long p0 = a.cum_pages[b], p1 = a.cum_pages[b + 1];
  int tok0 = b * a.q_len, nq = a.q_len;
  if (a.cu_q) {
    tok0 = a.cu_q[b];
    nq = a.cu_q[b + 1] - tok0;
  }
  if (row >= a.rows || row >= nq * a.heads) return;  // a row the request does not have
  if (p1 <= p0) return;
  const size_t orow = (size_t)tok0 * a.heads + row;
  const int G = a.grid;
  const int g0 = owner_group(p0, P, G), g1 = owner_group(p1 - 1, P, G);
  const int ns = g1 - g0 + 1;
  const float* lse_col = a.part_lse + (size_t)(g0 + b) * a.rows + row;
  const int col = quarter * (kDv / 4) + 4 * quad;
  const uint16_t* o_col = a.part_o + ((size_t)(g0 + b) * a.rows + row) * kDv + col;
  const size_t share_stride = (size_t)a.rows * kDv;
  const bool sparse = P < G;

  float m = -INFINITY, wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < ns; i0 += kMergeDepth) {
    float l[kMergeDepth];
    bf16x4 x[kMergeDepth];
#pragma unroll
    for (int u = 0; u < kMergeDepth; ++u) {
      const int i = i0 + u;
      const bool has = i < ns && (!sparse || !share_empty(P, G, g0 + i));
      l[u] = has ? lse_col[(size_t)i * a.rows] : -INFINITY;
      x[u] = *reinterpret_cast<const bf16x4*>(o_col + (size_t)(has ? i : 0) * share_stride);
    }
#pragma unroll
    for (int u = 0; u < kMergeDepth; ++u) {
      if (l[u] == -INFINITY) continue;
      if (l[u] > m) {
        const float r = fast_exp2(m - l[u]);  // 0 while nothing has been added
        acc *= r;
        wsum *= r;
        m = l[u];
      }
      const float wt = fast_exp2(l[u] - m);
      acc += f32x4{(float)x[u][0], (float)x[u][1], (float)x[u][2], (float)x[u][3]} * wt;
      wsum += wt;
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  bf16x4 h;
  h[0] = (__bf16)(acc[0] * inv); h[1] = (__bf16)(acc[1] * inv);
  h[2] = (__bf16)(acc[2] * inv); h[3] = (__bf16)(acc[3] * inv);
  *reinterpret_cast<bf16x4*>(a.out + orow * kDv + col) = h;
  if (quarter == 0 && quad == 0) a.lse[orow] = wsum > 0.f ? (m + fast_log2(wsum)) * kLn2 : -INFINITY;
}

// Split-KV scratch of the allocation-free decode entry point.  In host code `scratch`
// names a host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns for the current device is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};  // per device, kept until the process ends
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodePlan& plan, const DecodeArgs& args, int kv_dtype, hipStream_t stream) {
  const int row_blocks = (args.rows + kBlockRows - 1) / kBlockRows;
  if (kv_dtype == 1)
    hipLaunchKernelGGL(decode_ws_codes<kCodeInt8>, dim3(plan.grid, row_blocks), dim3(kWaves * 64), 0, stream, args);
  else if (kv_dtype == 2)
    hipLaunchKernelGGL(decode_ws_codes<kCodeFp8>, dim3(plan.grid, row_blocks), dim3(kWaves * 64), 0, stream, args);
  else
    hipLaunchKernelGGL(decode_phase1_pipe, dim3(plan.grid, row_blocks), dim3(kWaves * 64), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.grid == 1) return e;
  if (plan.grid <= kMergeRowsShares * args.batch) {
    const int row_blocks_m = (args.rows + kMergeRows - 1) / kMergeRows;
    hipLaunchKernelGGL(decode_merge_rows, dim3(args.batch * row_blocks_m, 4), dim3(256), 0, stream, args);
  } else {
    hipLaunchKernelGGL(decode_merge, dim3(args.batch * args.rows, 4), dim3(256), 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace mla
