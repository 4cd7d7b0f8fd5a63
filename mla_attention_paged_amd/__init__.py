"""Python binding of the MLA paged-attention library (gfx950 HIP kernels).

Argument marshalling only: every function here calls the C ABI declared in
``include/mla.h`` with the same name and the same argument order.  Pointer
arguments accept a torch tensor (its ``data_ptr()``), an integer address or
None; ``hip_stream`` accepts a ``torch.cuda.Stream``, an integer handle or
None (torch's current stream).  A non-zero status raises ``MLAError``.

The compute path runs only in the HIP library: when ``_build/libmla.so`` is
missing, every call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE = 3
MLA_ERR_HIP = 4
MLA_ERR_SCRATCH = 5
MLA_NOALLOC_SCRATCH_BYTES = 64 << 20
MLA_KV_BF16 = 0
MLA_KV_INT8 = 1
MLA_KV_FP8 = 2
MLA_DIM_QK = 576
MLA_DIM_V = 512
MLA_PAGE_SIZE = 64

_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mla_status_string(status)} (status {status})")


def library():
    """The loaded HIP library; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"MLA HIP library not built ({LIB_PATH} missing); "
                               "run __graft_entry__.build() or python -m mla_attention_paged_amd._build")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.mla_splitkv_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        lib.mla_splitkv_workspace_size.restype = i32
        lib.mla_decode.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, f32, vp, vp,
                                   vp, sz, vp]
        lib.mla_decode.restype = i32
        lib.mla_decode_noalloc.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, f32, vp, vp,
                                           vp]
        lib.mla_decode_noalloc.restype = i32
        lib.mla_decode_varlen.argtypes = [vp, vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32,
                                          vp, vp, vp, sz, vp]
        lib.mla_decode_varlen.restype = i32
        lib.mla_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, i32,
                                           f32, vp, vp, vp, sz, vp]
        lib.mla_prefill_varlen.restype = i32
        lib.mla_q_absorb.argtypes = [vp, vp, vp, i32, i32, vp]
        lib.mla_q_absorb.restype = i32
        lib.mla_v_up.argtypes = [vp, vp, vp, i32, i32, vp]
        lib.mla_v_up.restype = i32
        lib.mla_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, vp]
        lib.mla_kv_append.restype = i32
        lib.mla_status_string.argtypes = [i32]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_decode_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(sz)]
        lib.mla_decode_plan.restype = i32
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(s, int):
        return s or None
    return s.cuda_stream or None


def _check(rc: int, where: str) -> None:
    if rc != MLA_OK:
        raise MLAError(rc, where)


def mla_status_string(status: int) -> str:
    return library().mla_status_string(int(status)).decode()


def mla_splitkv_workspace_size(batch, num_heads, max_q_len, total_q, max_seq_len, kv_dtype) -> int:
    out = ctypes.c_size_t(0)
    _check(library().mla_splitkv_workspace_size(batch, num_heads, max_q_len, total_q, max_seq_len,
                                                kv_dtype, ctypes.byref(out)), "mla_splitkv_workspace_size")
    return int(out.value)


def mla_decode_plan(batch, num_heads, q_len, max_seq_len, kv_dtype, num_cus=0):
    """(phase-one workgroups, workspace bytes) of the decode split plan."""
    g = ctypes.c_int(0)
    b = ctypes.c_size_t(0)
    _check(library().mla_decode_plan(batch, num_heads, q_len, max_seq_len, kv_dtype, num_cus,
                                     ctypes.byref(g), ctypes.byref(b)), "mla_decode_plan")
    return int(g.value), int(b.value)


def mla_decode(q, kv_cache, kv_scale, kv_dtype, page_table, max_pages_per_req, seq_lens, batch, q_len,
               num_heads, page_size, max_seq_len, softmax_scale, out, lse, workspace, workspace_bytes,
               hip_stream=None) -> None:
    rc = library().mla_decode(_ptr(q), _ptr(kv_cache), _ptr(kv_scale), kv_dtype, _ptr(page_table),
                              max_pages_per_req, _ptr(seq_lens), batch, q_len, num_heads, page_size,
                              max_seq_len, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                              int(workspace_bytes), _stream(hip_stream))
    _check(rc, "mla_decode")


def mla_decode_noalloc(q, kv_cache, kv_scale, kv_dtype, page_table, max_pages_per_req, seq_lens, batch,
                       q_len, num_heads, page_size, max_seq_len, softmax_scale, out, lse, hip_stream=None) -> None:
    rc = library().mla_decode_noalloc(_ptr(q), _ptr(kv_cache), _ptr(kv_scale), kv_dtype, _ptr(page_table),
                                      max_pages_per_req, _ptr(seq_lens), batch, q_len, num_heads, page_size,
                                      max_seq_len, float(softmax_scale), _ptr(out), _ptr(lse), _stream(hip_stream))
    _check(rc, "mla_decode_noalloc")


def mla_decode_varlen(q, cu_seqlens_q, kv_cache, kv_scale, kv_dtype, page_table, max_pages_per_req, seq_lens,
                      batch, total_q, max_q_len, num_heads, page_size, max_seq_len, softmax_scale, out, lse,
                      workspace, workspace_bytes, hip_stream=None) -> None:
    rc = library().mla_decode_varlen(_ptr(q), _ptr(cu_seqlens_q), _ptr(kv_cache), _ptr(kv_scale), kv_dtype,
                                     _ptr(page_table), max_pages_per_req, _ptr(seq_lens), batch, total_q,
                                     max_q_len, num_heads, page_size, max_seq_len, float(softmax_scale),
                                     _ptr(out), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                     _stream(hip_stream))
    _check(rc, "mla_decode_varlen")


def mla_q_absorb(q, w_uk_t, q_out, tokens, num_heads, hip_stream=None) -> None:
    _check(library().mla_q_absorb(_ptr(q), _ptr(w_uk_t), _ptr(q_out), tokens, num_heads, _stream(hip_stream)),
           "mla_q_absorb")


def mla_v_up(o_lat, w_uv, out, tokens, num_heads, hip_stream=None) -> None:
    _check(library().mla_v_up(_ptr(o_lat), _ptr(w_uv), _ptr(out), tokens, num_heads, _stream(hip_stream)),
           "mla_v_up")


def mla_prefill_varlen(q, cu_seqlens_q, prefix_lens, kv_cache, kv_scale, kv_dtype, page_table,
                       max_pages_per_req, batch, total_q, max_q_len, max_seq_len, num_heads, page_size,
                       softmax_scale, out, lse, workspace, workspace_bytes, hip_stream=None) -> None:
    rc = library().mla_prefill_varlen(_ptr(q), _ptr(cu_seqlens_q), _ptr(prefix_lens), _ptr(kv_cache),
                                      _ptr(kv_scale), kv_dtype, _ptr(page_table), max_pages_per_req, batch,
                                      total_q, max_q_len, max_seq_len, num_heads, page_size,
                                      float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                      int(workspace_bytes), _stream(hip_stream))
    _check(rc, "mla_prefill_varlen")


def mla_kv_append(kv_new, cu_seqlens_new, start_pos, kv_cache, kv_scale, kv_dtype, page_table,
                  max_pages_per_req, batch, total_new, page_size, hip_stream=None) -> None:
    rc = library().mla_kv_append(_ptr(kv_new), _ptr(cu_seqlens_new), _ptr(start_pos), _ptr(kv_cache),
                                 _ptr(kv_scale), kv_dtype, _ptr(page_table), max_pages_per_req, batch,
                                 total_new, page_size, _stream(hip_stream))
    _check(rc, "mla_kv_append")
