"""Seeded synthetic inputs for MLA attention over a paged latent cache.

Serves both sides of every parity test and the benchmark.  It holds none of
the attention arithmetic: it draws request lengths, a page permutation, query
rows and latent cache rows, rounds them to bf16, and for the INT8 cache
applies the symmetric per-row quantisation that produces the stored int8
codes and their fp32 scales (the codes and scales are the inputs; how they
were produced does not enter any comparison).

Recipe (all deterministic from one integer seed):
  1. ``rng = numpy.random.default_rng(seed)`` draws the lengths (uniform
     integers, both ends inclusive), then ``rng.permutation`` of the page
     pool (all pages of all requests plus one poison page).
  2. Query rows and cache rows are i.i.d. N(0, 1) float32, drawn in fixed
     chunks, chunk ``c`` of stream ``s`` from
     ``default_rng(SeedSequence([seed, s, c]))`` (s = 1 for the cache in
     logical page order, s = 2 for the query in token order), so that threads
     can fill chunks in parallel without changing the values.
  3. bf16 values are round-to-nearest-even of the float32 draws.
  4. INT8: per 576-wide row, scale = max|x| / 127 in fp32, code =
     clip(rint(x / scale), -127, 127).
  4b. FP8 (E4M3 codes, uint8): per row, the codes are |x| * 64 truncated
     onto the E4M3 grid (3 mantissa bits; magnitudes below 2^-6 become 0,
     above 448 become 448; the sign of x in bit 7), and the fp32 scale is
     2^-6 * (1 + |x_0| / 16) with x_0 the row's first draw.  This is a
     generator recipe only: it is not the rounding of the append step, and
     the codes and scales are simply the inputs.
  5. Slots past a request's length in its last page, and the poison page that
     every unused page-table entry points at, hold a poison value (bf16
     1000.0 by default, optionally NaN).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

D_QK = 576          # latent 512 + rope 64: one cache row, and one query row
D_V = 512           # values are the first 512 columns of the same row
PAGE_SIZE = 64
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)

POISON_FINITE = 1000.0
POISON_NAN = float("nan")

_CACHE_CHUNK_PAGES = 128
_Q_CHUNK_TOKENS = 256


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + r) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_int8_rows(x: np.ndarray):
    """Symmetric per-row INT8: scale = max|x|/127 (fp32), code = clip(rint(x/scale), -127, 127)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    scale = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    codes = np.clip(np.rint(x / scale[..., None]), -127, 127).astype(np.int8)
    return codes, scale


def fp8_codes_from_draws(x: np.ndarray):
    """Recipe 4b: E4M3 code bytes and per-row scales from float32 draws [..., 576]."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64) * 64.0
    _, ex = np.frexp(a)
    E = ex - 1                                   # a in [2^E, 2^(E+1))
    m = np.floor((a / np.ldexp(1.0, E) - 1.0) * 8.0).astype(np.int64)
    e = E.astype(np.int64) + 7
    big = (e > 15) | ((e == 15) & (m == 7))
    e = np.where(big, 15, e)
    m = np.where(big, 6, m)
    mag = np.where(e >= 1, (e << 3) | m, 0)
    codes = (mag | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)
    scale = (np.float32(2.0 ** -6) * (np.float32(1.0) + np.abs(x[..., 0]) / np.float32(16.0))).astype(np.float32)
    return codes, scale


def _normal_chunks(seed: int, stream: int, shape_rows: int, row_shape: tuple, chunk: int,
                   sink) -> None:
    """Fill rows [0, shape_rows) chunk by chunk; ``sink(r0, r1, values_f32)`` stores each chunk."""
    nchunks = (shape_rows + chunk - 1) // chunk

    def work(c: int) -> None:
        r0 = c * chunk
        r1 = min(shape_rows, r0 + chunk)
        g = np.random.default_rng(np.random.SeedSequence([seed, stream, c]))
        sink(r0, r1, g.standard_normal((r1 - r0,) + row_shape, dtype=np.float32))

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
        return
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(work, range(nchunks)))


@dataclass
class PagedCache:
    """A paged latent cache as the kernels see it."""
    kv_dtype: str                 # "bf16", "int8" or "fp8"
    data: np.ndarray              # uint16 bf16 bits, int8 or uint8 E4M3 codes, [num_pages, page_size, 576]
    scale: Optional[np.ndarray]   # float32 [num_pages, page_size] for int8 and fp8, else None
    page_table: np.ndarray        # int32 [batch, max_pages]
    kv_lens: np.ndarray           # int32 [batch]: cached rows per request, new tokens included
    poison_page: int
    page_size: int = PAGE_SIZE

    @property
    def num_pages(self) -> int:
        return int(self.data.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def kv_bytes(self) -> int:
        """Bytes of the rows the requests actually hold (what attention must read)."""
        per_row = D_QK * 2 if self.kv_dtype == "bf16" else D_QK + 4
        return int(self.kv_lens.astype(np.int64).sum()) * per_row


def build_paged_cache(rng: np.random.Generator, seed: int, kv_lens, kv_dtype: str = "bf16",
                      max_pages: Optional[int] = None, poison: float = POISON_FINITE,
                      page_size: int = PAGE_SIZE) -> PagedCache:
    """Draw the page permutation from ``rng`` and fill every page (see the module recipe)."""
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    batch = kv_lens.shape[0]
    npages_b = [(int(L) + page_size - 1) // page_size for L in kv_lens]
    total = int(sum(npages_b))
    pool = total + 1
    if max_pages is None:
        max_pages = max([1] + npages_b)
    assert max_pages >= max([0] + npages_b)
    perm = rng.permutation(pool).astype(np.int32)
    poison_page = int(perm[total])
    page_table = np.full((batch, max_pages), poison_page, dtype=np.int32)
    logical_owner = np.empty((total, 2), dtype=np.int64)   # (request, page index) per logical page
    off = 0
    for b, n in enumerate(npages_b):
        page_table[b, :n] = perm[off:off + n]
        logical_owner[off:off + n, 0] = b
        logical_owner[off:off + n, 1] = np.arange(n)
        off += n

    if kv_dtype == "bf16":
        data = np.empty((pool, page_size, D_QK), dtype=np.uint16)
        scale = None
    elif kv_dtype in ("int8", "fp8"):
        data = np.empty((pool, page_size, D_QK), dtype=np.int8 if kv_dtype == "int8" else np.uint8)
        scale = np.empty((pool, page_size), dtype=np.float32)
    else:
        raise ValueError(f"unknown kv dtype {kv_dtype!r}")

    def sink(r0: int, r1: int, x: np.ndarray) -> None:
        phys = perm[r0:r1]
        if kv_dtype == "bf16":
            data[phys] = bf16_bits(x)
        else:
            codes, s = quantize_int8_rows(x) if kv_dtype == "int8" else fp8_codes_from_draws(x)
            data[phys] = codes
            scale[phys] = s

    _normal_chunks(seed, 1, total, (page_size, D_QK), _CACHE_CHUNK_PAGES, sink)

    # Poison: the unused tail of each request's last page, and the poison page.
    if kv_dtype == "bf16":
        pbits = bf16_bits(np.array([poison], dtype=np.float32))[0]
        data[poison_page] = pbits
    else:
        pcode = 127 if kv_dtype == "int8" else 0x7E   # the largest code: 127, or E4M3 448
        data[poison_page] = pcode
        scale[poison_page] = np.float32(poison)
    for b in range(batch):
        L = int(kv_lens[b])
        n = npages_b[b]
        used = L - (n - 1) * page_size if n else 0
        if n and used < page_size:
            pg = page_table[b, n - 1]
            if kv_dtype == "bf16":
                data[pg, used:] = pbits
            else:
                data[pg, used:] = pcode
                scale[pg, used:] = np.float32(poison)
    return PagedCache(kv_dtype, data, scale, page_table, kv_lens, poison_page, page_size)


def draw_query(seed: int, tokens: int, heads: int) -> np.ndarray:
    """bf16 bits of i.i.d. N(0,1) query rows, [tokens, heads, 576]."""
    q = np.empty((tokens, heads, D_QK), dtype=np.uint16)

    def sink(r0, r1, x):
        q[r0:r1] = bf16_bits(x)

    _normal_chunks(seed, 2, tokens, (heads, D_QK), _Q_CHUNK_TOKENS, sink)
    return q


@dataclass
class DecodeCase:
    """Inputs of one decode call: ``q_len`` new tokens per request, folded with the heads."""
    batch: int
    heads: int
    q_len: int
    q: np.ndarray                 # uint16 [batch*q_len, heads, 576]
    cache: PagedCache
    max_seq_len: int
    softmax_scale: float = DEFAULT_SCALE
    name: str = ""

    @property
    def seq_lens(self) -> np.ndarray:
        return self.cache.kv_lens

    def q_start(self) -> np.ndarray:
        return (np.arange(self.batch + 1, dtype=np.int32) * self.q_len).astype(np.int32)

    def total_q(self) -> int:
        return self.batch * self.q_len


@dataclass
class PrefillCase:
    """Inputs of one varlen prefill call (no padding, cu_seqlens layout)."""
    heads: int
    q: np.ndarray                 # uint16 [total_q, heads, 576]
    cu_seqlens_q: np.ndarray      # int32 [batch+1]
    prefix_lens: np.ndarray       # int32 [batch]
    cache: PagedCache             # kv_lens = prefix + new
    max_seq_len: int
    softmax_scale: float = DEFAULT_SCALE
    name: str = ""

    @property
    def batch(self) -> int:
        return int(self.prefix_lens.shape[0])

    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    def max_q_len(self) -> int:
        return int(np.diff(self.cu_seqlens_q).max()) if self.batch else 0


def make_decode_case(seed: int, batch: int, heads: int, q_len: int, seq_lens=None,
                     len_range=None, kv_dtype: str = "bf16", max_seq_len: Optional[int] = None,
                     poison: float = POISON_FINITE, name: str = "", page_size: int = PAGE_SIZE) -> DecodeCase:
    """Decode inputs.  Lengths are ``seq_lens`` or drawn uniformly from ``len_range`` (inclusive)."""
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        lo, hi = len_range
        seq_lens = rng.integers(lo, hi, size=batch, endpoint=True)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (batch,) and (seq_lens >= q_len).all()
    if max_seq_len is None:
        max_seq_len = int(len_range[1]) if len_range is not None else int(seq_lens.max())
    max_pages = (max_seq_len + page_size - 1) // page_size
    cache = build_paged_cache(rng, seed, seq_lens, kv_dtype, max_pages=max_pages, poison=poison,
                              page_size=page_size)
    q = draw_query(seed, batch * q_len, heads)
    return DecodeCase(batch, heads, q_len, q, cache, max_seq_len, DEFAULT_SCALE, name)


def make_prefill_case(seed: int, heads: int, prefix_lens=None, new_lens=None, batch: int = 0,
                      prefix_range=None, new_range=None, kv_dtype: str = "bf16",
                      poison: float = POISON_FINITE, name: str = "", page_size: int = PAGE_SIZE) -> PrefillCase:
    """Varlen prefill inputs: request b has prefix_lens[b] cached rows plus new_lens[b] new ones."""
    rng = np.random.default_rng(seed)
    if prefix_lens is None:
        prefix_lens = rng.integers(prefix_range[0], prefix_range[1], size=batch, endpoint=True)
    if new_lens is None:
        new_lens = rng.integers(new_range[0], new_range[1], size=len(prefix_lens), endpoint=True)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int32)
    new_lens = np.asarray(new_lens, dtype=np.int32)
    kv_lens = (prefix_lens + new_lens).astype(np.int32)
    cu = np.zeros(len(new_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(new_lens)
    max_seq_len = int(kv_lens.max()) if len(kv_lens) else 1
    max_pages = max(1, (max_seq_len + page_size - 1) // page_size)
    cache = build_paged_cache(rng, seed, kv_lens, kv_dtype, max_pages=max_pages, poison=poison,
                              page_size=page_size)
    q = draw_query(seed, int(cu[-1]), heads)
    return PrefillCase(heads, q, cu, prefix_lens, cache, max_seq_len, DEFAULT_SCALE, name)


# The five benchmark workloads; configuration k is drawn with seed k + 1.
WORKLOADS = {
    0: dict(name="decode_b1_h16_q1_L256", kind="decode", batch=1, heads=16, q_len=1,
            seq_lens=[256], kv_dtype="bf16"),
    1: dict(name="decode_b4_h16_q4_L64K", kind="decode", batch=4, heads=16, q_len=4,
            seq_lens=[65536] * 4, kv_dtype="bf16"),
    2: dict(name="decode_b16_h32_q2_L32K-128K", kind="decode", batch=16, heads=32, q_len=2,
            len_range=(32768, 131072), kv_dtype="bf16"),
    3: dict(name="prefill_b8_h16_P16K-96K_N200-2000", kind="prefill", batch=8, heads=16,
            prefix_range=(16384, 98304), new_range=(200, 2000), kv_dtype="bf16"),
    4: dict(name="decode_int8_b8_h16_q4_L256K", kind="decode", batch=8, heads=16, q_len=4,
            seq_lens=[262144] * 8, kv_dtype="int8"),
}


def make_workload(k: int, poison: float = POISON_FINITE):
    """Benchmark workload ``k`` (0..4), seed k + 1."""
    w = WORKLOADS[k]
    seed = k + 1
    if w["kind"] == "decode":
        return make_decode_case(seed, w["batch"], w["heads"], w["q_len"], seq_lens=w.get("seq_lens"),
                                len_range=w.get("len_range"), kv_dtype=w["kv_dtype"],
                                poison=poison, name=w["name"])
    return make_prefill_case(seed, w["heads"], batch=w["batch"], prefix_range=w["prefix_range"],
                             new_range=w["new_range"], kv_dtype=w["kv_dtype"], poison=poison,
                             name=w["name"])
