"""fp64 CPU oracle for MLA attention over a paged latent cache (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library's compute path never does.

``mla_oracle.c`` holds the definition (see its header for the passages it
follows); this module compiles it with gcc when the shared object is missing
or older than the source, and wraps it with ctypes.  ``kv_append.py`` is the
oracle of the step that writes new tokens' rows into the pages; ``absorb.py``
that of the query absorption and value up-projection around the attention.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libmla_oracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_dblp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, -O2, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(_LIB), exist_ok=True)
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """ctypes handle for an oracle shared object (the default one unless a path is given)."""
    lib = ctypes.CDLL(path)
    common = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
              _i32p, ctypes.c_int, ctypes.c_int, _i32p, _i32p, ctypes.c_int, ctypes.c_int,
              ctypes.c_int, ctypes.c_int, ctypes.c_double]
    lib.mla_oracle_attention.argtypes = common + [_i32p, ctypes.c_int, _dblp, _dblp, ctypes.c_int]
    lib.mla_oracle_attention.restype = ctypes.c_int
    lib.mla_oracle_attention_split.argtypes = common + [_i32p, ctypes.c_int, _i32p, ctypes.c_int,
                                                        _dblp, _dblp, ctypes.c_int]
    lib.mla_oracle_attention_split.restype = ctypes.c_int
    lib.mla_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.mla_oracle_e4m3_value.restype = ctypes.c_double
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = load_library(_LIB)
    return _lib


def _ptr(a: Optional[np.ndarray], typ=None):
    if a is None:
        return None
    if typ is None:
        return a.ctypes.data_as(ctypes.c_void_p)
    return a.ctypes.data_as(typ)


def default_threads() -> int:
    return max(1, os.cpu_count() or 1)


def attention(q_bits: np.ndarray, cache: np.ndarray, kv_scale: Optional[np.ndarray],
              page_table: np.ndarray, q_start: np.ndarray, kv_len: np.ndarray,
              softmax_scale: float, dv: int = 512, tokens=None, bounds=None,
              nthreads: Optional[int] = None, lib=None):
    """Attention for the given query tokens (all tokens when ``tokens`` is None).

    q_bits: uint16 bf16 bits [total_q, H, dqk]; cache: uint16 bf16 bits, int8
    codes or uint8 E4M3 codes [num_pages, page_size, dqk]; kv_scale: float32
    [num_pages, page_size] for int8 and fp8; page_table int32 [batch, max_pages]; q_start int32 [batch+1];
    kv_len int32 [batch].  ``bounds`` selects the split form.  Returns
    (out float64 [n, H, dv], lse float64 [n, H]).
    """
    lib = lib or _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    if cache.dtype in (np.int8, np.uint8):
        kind = 1 if cache.dtype == np.int8 else 2
        cache = np.ascontiguousarray(cache)
        if kv_scale is None:
            raise ValueError("int8 / fp8 cache needs kv_scale")
        kv_scale = np.ascontiguousarray(kv_scale, dtype=np.float32)
    else:
        kind = 0
        cache = np.ascontiguousarray(cache, dtype=np.uint16)
        kv_scale = None
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    q_start = np.ascontiguousarray(q_start, dtype=np.int32)
    kv_len = np.ascontiguousarray(kv_len, dtype=np.int32)
    total_q, H, dqk = q_bits.shape
    num_pages, page_size, dqk2 = cache.shape
    assert dqk2 == dqk
    batch = kv_len.shape[0]
    assert q_start.shape == (batch + 1,) and page_table.shape[0] == batch
    if tokens is None:
        tok = None
        n = int(q_start[-1])
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = tok.shape[0]
    out = np.zeros((n, H, dv), dtype=np.float64)
    lse = np.zeros((n, H), dtype=np.float64)
    nt = nthreads or default_threads()
    args = [_ptr(q_bits), kind, _ptr(cache), _ptr(kv_scale), num_pages, _ptr(page_table, _i32p),
            page_table.shape[1], page_size, _ptr(q_start, _i32p), _ptr(kv_len, _i32p), batch, H,
            dqk, dv, float(softmax_scale)]
    if bounds is None:
        rc = lib.mla_oracle_attention(*args, _ptr(tok, _i32p), n, _ptr(out, _dblp), _ptr(lse, _dblp), nt)
    else:
        b = np.ascontiguousarray(bounds, dtype=np.int32)
        rc = lib.mla_oracle_attention_split(*args, _ptr(b, _i32p), b.shape[0] - 1, _ptr(tok, _i32p), n,
                                            _ptr(out, _dblp), _ptr(lse, _dblp), nt)
    if rc != 0:
        raise ValueError(f"oracle rejected its inputs (code {rc})")
    return out, lse


def decode(case, tokens=None, bounds=None, nthreads=None):
    """Oracle for a ``synth.DecodeCase`` (token b*q_len + i is draft i of request b)."""
    c = case.cache
    return attention(case.q, c.data, c.scale, c.page_table, case.q_start(), c.kv_lens,
                     case.softmax_scale, tokens=tokens, bounds=bounds, nthreads=nthreads)


def prefill(case, tokens=None, bounds=None, nthreads=None):
    """Oracle for a ``synth.PrefillCase``."""
    c = case.cache
    return attention(case.q, c.data, c.scale, c.page_table, case.cu_seqlens_q, c.kv_lens,
                     case.softmax_scale, tokens=tokens, bounds=bounds, nthreads=nthreads)


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code byte, as the attention oracle decodes it."""
    return float(_load().mla_oracle_e4m3_value(int(code) & 0xFF))


from .kv_append import kv_append, quantize_row, quantize_row_fp8, e4m3_round  # noqa: E402
from . import absorb  # noqa: E402  (the products on either side of the absorbed attention)
