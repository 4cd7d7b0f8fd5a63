"""Oracle for writing new tokens' rows into the paged latent cache (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this module; the library's compute path never does.

What it follows.  [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎", section
"Kernel：让 MLA 真正跑满 GPU": attention runs over a paged cache of compressed
latent rows, one row per token, and an INT8 latent cache is one way to cut the
bandwidth decode needs.  The cache layout and the INT8 encoding are the ones
the attention entry points read: page ``page_table[b][t // 64]``, slot
``t % 64`` for logical position ``t`` of request ``b``; an INT8 row is
576 codes plus one fp32 scale, value = code * scale, symmetric, per row.

The quantisation is written out as its definition, in fp32 as the cache stores
it: scale = max|x| / 127 (an all-zero row gets scale 1), code =
clip(rint(x / scale), -127, 127) with numpy's round-half-even ``rint``.
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


def kv_append(kv_new_bits: np.ndarray, cu_seqlens_new: np.ndarray, start_pos: np.ndarray,
              cache: np.ndarray, kv_scale: Optional[np.ndarray], kv_dtype: str,
              page_table: np.ndarray, quantize=quantize_row) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Return copies of ``cache`` (and ``kv_scale``) with the new rows written.

    kv_new_bits: uint16 bf16 bits [total_new, 576]; cache: [num_pages, 64, 576]
    (uint16 bf16 bits, or int8 codes with kv_scale float32 [num_pages, 64]).
    Row j of request b goes to logical position start_pos[b] + j; positions
    outside the request's page table are not written.
    """
    out = np.array(cache, copy=True)
    sc = None if kv_scale is None else np.array(kv_scale, copy=True)
    max_pages = page_table.shape[1]
    batch = len(start_pos)
    for b in range(batch):
        for j in range(int(cu_seqlens_new[b + 1]) - int(cu_seqlens_new[b])):
            t = int(start_pos[b]) + j
            if t < 0 or t >= max_pages * 64:
                continue
            page, slot = int(page_table[b, t // 64]), t % 64
            row = kv_new_bits[int(cu_seqlens_new[b]) + j]
            if kv_dtype == "bf16":
                out[page, slot] = row
            else:
                codes, scale = quantize(bf16_bits_to_f32(row))
                out[page, slot] = codes
                sc[page, slot] = scale
    return out, sc
