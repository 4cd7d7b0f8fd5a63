"""Oracle for writing new tokens' rows into the paged latent cache (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this module; the library's compute path never does.

What it follows.  [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎", section
"Kernel：让 MLA 真正跑满 GPU": attention runs over a paged cache of compressed
latent rows, one row per token, and an INT8 latent cache is one way to cut the
bandwidth decode needs.  The cache layout and the INT8 encoding are the ones
the attention entry points read: page ``page_table[b][t // page_size]``, slot
``t % page_size`` for logical position ``t`` of request ``b`` (the page size is
the cache's second dimension); an INT8 row is
576 codes plus one fp32 scale, value = code * scale, symmetric, per row.

The quantisation is written out as its definition, in fp32 as the cache stores
it: scale = max|x| / 127 (an all-zero row gets scale 1), code =
clip(rint(x / scale), -127, 127) with numpy's round-half-even ``rint``.

FP8 cache ([GITREAD] "TokenSpeed 深度解析:把 LLM 推理压到"光速"意味着什么",
section "核心技术揭秘": FP8 KV-cache quantisation is standard; no format is
given).  Read as OCP E4M3 (finite variant; largest magnitude 448) with the
same per-row fp32 scale: scale = max|x| / 448 in fp32 (an all-zero row gets
scale 1), then x / scale in fp32 is rounded to the nearest E4M3 value, ties
to the even mantissa, magnitudes above 448 saturating to 448 (the division
never exceeds 448 by more than an fp32 rounding, so this only guards).
Plain loops over requests, numpy per row; no blocking or reordering.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_row(x: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """Symmetric INT8 codes and fp32 scale of one row of float32 values."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x)))
    scale = np.float32(amax / np.float32(127.0))
    if scale == np.float32(0.0):
        scale = np.float32(1.0)
    codes = np.clip(np.rint(x / scale), -127, 127).astype(np.int8)
    return codes, scale


E4M3_MAX = 448.0


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """E4M3 code bytes (uint8) of float32 values: nearest value, ties to even.

    The grid at magnitude a is 2^(E-3) for a in [2^E, 2^(E+1)), E >= -6 (the
    normal binades), and 2^-9 below 2^-6 (the subnormals).  Rounding a / grid
    to the nearest integer with ties to even (numpy ``rint``, exact in
    float64 because the grid is a power of two) is rounding the mantissa to
    3 bits.  The code of the rounded magnitude r is then e = E' + 7, m =
    8 (r / 2^E' - 1) for a normal r in [2^E', 2^(E'+1)), and e = 0, m =
    r / 2^-9 for a subnormal one; the sign goes to bit 7.
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1): a in [2^(ex-1), 2^ex)
    E = np.maximum(ex - 1, -6)
    grid = np.ldexp(1.0, E - 3)
    r = np.minimum(np.rint(a / grid) * grid, E4M3_MAX)
    _, ex2 = np.frexp(r)
    E2 = ex2 - 1
    normal = r >= 2.0 ** -6
    e = np.where(normal, E2 + 7, 0)
    m = np.where(normal, (r / np.ldexp(1.0, E2) - 1.0) * 8.0, r / 2.0 ** -9)
    code = (e.astype(np.int64) << 3) | np.rint(m).astype(np.int64)
    code = np.where(r == 0.0, 0, code)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def quantize_row_fp8(x: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """E4M3 codes and fp32 scale of one row of float32 values."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x)))
    scale = np.float32(amax / np.float32(E4M3_MAX))
    if scale == np.float32(0.0):
        scale = np.float32(1.0)
    return e4m3_round(x / scale), scale


def kv_append(kv_new_bits: np.ndarray, cu_seqlens_new: np.ndarray, start_pos: np.ndarray,
              cache: np.ndarray, kv_scale: Optional[np.ndarray], kv_dtype: str,
              page_table: np.ndarray, quantize=quantize_row,
              quantize_fp8=quantize_row_fp8) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Return copies of ``cache`` (and ``kv_scale``) with the new rows written.

    kv_new_bits: uint16 bf16 bits [total_new, 576]; cache: [num_pages, page_size, 576]
    (uint16 bf16 bits, or int8 / uint8 E4M3 codes with kv_scale float32
    [num_pages, page_size]); kv_dtype "bf16", "int8" or "fp8".  ``quantize``
    replaces the INT8 quantiser, ``quantize_fp8`` the FP8 one.
    Row j of request b goes to logical position start_pos[b] + j; positions
    outside the request's page table are not written.
    """
    out = np.array(cache, copy=True)
    sc = None if kv_scale is None else np.array(kv_scale, copy=True)
    max_pages = page_table.shape[1]
    page_size = cache.shape[1]
    batch = len(start_pos)
    for b in range(batch):
        for j in range(int(cu_seqlens_new[b + 1]) - int(cu_seqlens_new[b])):
            t = int(start_pos[b]) + j
            if t < 0 or t >= max_pages * page_size:
                continue
            page, slot = int(page_table[b, t // page_size]), t % page_size
            row = kv_new_bits[int(cu_seqlens_new[b]) + j]
            if kv_dtype == "bf16":
                out[page, slot] = row
            else:
                q = quantize if kv_dtype == "int8" else quantize_fp8
                codes, scale = q(bf16_bits_to_f32(row))
                out[page, slot] = codes
                sc[page, slot] = scale
    return out, sc
