"""The C-ABI library on the host: it loads, exports what include/mla.h declares,
and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import mla_attention_paged_amd as mla
from mla_attention_paged_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        _build.build()
    os.environ["MLA_NUM_CUS"] = "256"
    return mla.library()


def _declared():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"mla_decode", "mla_prefill_varlen", "mla_splitkv_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(6):
        assert mla.mla_status_string(code) not in ("", "unknown status")
    assert mla.mla_status_string(99) == "unknown status"


def _decode_rc(lib, **kw):
    a = dict(q=1, kv=1, scale=None, kind=0, pt=1, maxp=1024, lens=1, batch=4, q_len=4, heads=16, page=64,
             maxlen=65536, scale_f=0.07, out=1, lse=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.mla_decode(a["q"], a["kv"], a["scale"], a["kind"], a["pt"], a["maxp"], a["lens"], a["batch"],
                          a["q_len"], a["heads"], a["page"], a["maxlen"], a["scale_f"], a["out"], a["lse"],
                          a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), mla.MLA_ERR_INVALID),
    (dict(kv=None), mla.MLA_ERR_INVALID),
    (dict(pt=None), mla.MLA_ERR_INVALID),
    (dict(lens=None), mla.MLA_ERR_INVALID),
    (dict(out=None), mla.MLA_ERR_INVALID),
    (dict(lse=None), mla.MLA_ERR_INVALID),
    (dict(batch=0), mla.MLA_ERR_INVALID),
    (dict(q_len=0), mla.MLA_ERR_INVALID),
    (dict(heads=0), mla.MLA_ERR_INVALID),
    (dict(page=32), mla.MLA_ERR_UNSUPPORTED),
    (dict(page=96), mla.MLA_ERR_UNSUPPORTED),       # not a whole number of 64-row sub-pages
    (dict(page=8192), mla.MLA_ERR_UNSUPPORTED),     # above the largest page size
    (dict(page=128), mla.MLA_ERR_WORKSPACE),        # supported: reaches the workspace check
    (dict(page=1536, maxp=43), mla.MLA_ERR_WORKSPACE),
    (dict(page=1536, maxp=42), mla.MLA_ERR_INVALID),  # 42 * 1536 rows < max_seq_len
    (dict(kind=3), mla.MLA_ERR_UNSUPPORTED),
    (dict(kind=1), mla.MLA_ERR_INVALID),            # int8 without scales
    (dict(kind=2), mla.MLA_ERR_INVALID),            # fp8 without scales
    (dict(q_len=9, heads=16), mla.MLA_ERR_UNSUPPORTED),  # 144 folded rows
    (dict(scale_f=0.0), mla.MLA_ERR_INVALID),
    (dict(scale_f=float("nan")), mla.MLA_ERR_INVALID),
    (dict(maxlen=3), mla.MLA_ERR_INVALID),          # shorter than q_len
    (dict(maxp=1023), mla.MLA_ERR_INVALID),         # table narrower than max_seq_len
    (dict(ws=8), mla.MLA_ERR_INVALID),              # misaligned workspace
    (dict(ws=None, wsb=0), mla.MLA_ERR_WORKSPACE),  # plan needs a workspace
])
def test_decode_argument_checks(lib, kw, code):
    assert _decode_rc(lib, **kw) == code


def test_prefill_argument_checks(lib):
    def rc(**kw):
        a = dict(q=1, cu=1, prefix=1, kv=1, scale=None, kind=0, pt=1, maxp=64, batch=2, tq=10, mq=6, maxlen=4096,
                 heads=16, page=64, sf=0.07, out=1, lse=1, ws=None, wsb=0)
        a.update(kw)
        return lib.mla_prefill_varlen(a["q"], a["cu"], a["prefix"], a["kv"], a["scale"], a["kind"], a["pt"],
                                      a["maxp"], a["batch"], a["tq"], a["mq"], a["maxlen"], a["heads"], a["page"],
                                      a["sf"], a["out"], a["lse"], a["ws"], a["wsb"], None)
    assert rc(cu=None) == mla.MLA_ERR_INVALID
    assert rc(prefix=None) == mla.MLA_ERR_INVALID
    assert rc(heads=129) == mla.MLA_ERR_UNSUPPORTED
    assert rc(kind=2) == mla.MLA_ERR_INVALID             # fp8 without scales
    assert rc(kind=3) == mla.MLA_ERR_UNSUPPORTED
    assert rc(page=16) == mla.MLA_ERR_UNSUPPORTED
    assert rc(tq=5, mq=6) == mla.MLA_ERR_INVALID
    assert rc(maxp=63) == mla.MLA_ERR_INVALID
    assert rc(ws=None) == mla.MLA_ERR_WORKSPACE
    assert rc(tq=0, mq=0) == mla.MLA_OK                # nothing to do, no launch


def test_decode_plan_shapes(lib):
    # 64K-row decode, 4 requests: one phase-one workgroup per compute unit
    g, ws = mla.mla_decode_plan(4, 16, 4, 65536, 0, num_cus=256)
    assert g == 256 and ws >= (256 + 4) * 64 * (512 * 2 + 4)  # bf16 partial outputs + fp32 log2-sum-exp
    # 256 rows (four pages): one workgroup per page, partials and a merge
    g, ws = mla.mla_decode_plan(1, 16, 1, 256, 0, num_cus=256)
    assert g == 4 and ws >= (4 + 1) * 16 * (512 * 2 + 4)
    # one page: a single workgroup writes the output directly, no workspace
    assert mla.mla_decode_plan(1, 16, 1, 64, 0, num_cus=256) == (1, 0)
    # at least one page per workgroup, at most one workgroup per compute unit
    g, _ = mla.mla_decode_plan(2, 16, 1, 640, 0, num_cus=256)
    assert g == 20
    g, _ = mla.mla_decode_plan(2, 16, 1, 640, 0, num_cus=8)
    assert g == 8
    # more rows per request (q_len * heads > 64): two row blocks per share, half the shares,
    # so that the grid is still one workgroup per compute unit
    g, ws = mla.mla_decode_plan(2, 32, 4, 8192, 0, num_cus=256)
    assert g == 128 and ws > 0


def test_workspace_size_is_monotone_and_covers_plan(lib):
    prev = 0
    for L in (64, 256, 1024, 8192, 65536, 262144):
        ws = mla.mla_splitkv_workspace_size(4, 16, 4, 16, L, 0)
        assert ws >= prev
        assert ws >= mla.mla_decode_plan(4, 16, 4, L, 0, num_cus=256)[1]
        prev = ws
    # prefill shapes need only the small work-list area
    assert 0 < mla.mla_splitkv_workspace_size(8, 16, 2000, 8629, 100304, 0) < 1 << 20


def test_workspace_size_argument_checks(lib):
    out = ctypes.c_size_t(0)
    assert lib.mla_splitkv_workspace_size(4, 16, 4, 16, 1024, 0, None) == mla.MLA_ERR_INVALID
    assert lib.mla_splitkv_workspace_size(0, 16, 4, 16, 1024, 0, ctypes.byref(out)) == mla.MLA_ERR_INVALID
    assert lib.mla_splitkv_workspace_size(4, 16, 4, -1, 1024, 0, ctypes.byref(out)) == mla.MLA_ERR_INVALID
    assert lib.mla_splitkv_workspace_size(4, 16, 4, 3, 1024, 0, ctypes.byref(out)) == mla.MLA_OK  # ragged decode
    assert lib.mla_splitkv_workspace_size(4, 16, 4, 16, 1024, 7, ctypes.byref(out)) == mla.MLA_ERR_UNSUPPORTED
    assert lib.mla_splitkv_workspace_size(4, 16, 4, 16, 1024, 2, ctypes.byref(out)) == mla.MLA_OK


def _append_rc(lib, **kw):
    a = dict(new=1, cu=1, start=1, kv=1, scale=None, kind=0, pt=1, maxp=16, batch=2, total=8, page=64,
             stream=None)
    a.update(kw)
    return lib.mla_kv_append(a["new"], a["cu"], a["start"], a["kv"], a["scale"], a["kind"], a["pt"],
                             a["maxp"], a["batch"], a["total"], a["page"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(new=None), mla.MLA_ERR_INVALID),
    (dict(cu=None), mla.MLA_ERR_INVALID),
    (dict(start=None), mla.MLA_ERR_INVALID),
    (dict(kv=None), mla.MLA_ERR_INVALID),
    (dict(pt=None), mla.MLA_ERR_INVALID),
    (dict(batch=0), mla.MLA_ERR_INVALID),
    (dict(total=-1), mla.MLA_ERR_INVALID),
    (dict(maxp=0), mla.MLA_ERR_INVALID),
    (dict(kind=1), mla.MLA_ERR_INVALID),            # int8 without scales
    (dict(kind=2), mla.MLA_ERR_INVALID),            # fp8 without scales
    (dict(kind=3), mla.MLA_ERR_UNSUPPORTED),
    (dict(page=96), mla.MLA_ERR_UNSUPPORTED),
    (dict(total=0, new=None, kv=None), mla.MLA_OK),  # nothing to write, nothing enqueued
])
def test_append_argument_checks(lib, kw, code):
    assert _append_rc(lib, **kw) == code


def _varlen_rc(lib, **kw):
    a = dict(q=1, cu=1, kv=1, scale=None, kind=0, pt=1, maxp=1024, lens=1, batch=4, tq=10, mq=4, heads=16,
             page=64, maxlen=65536, sf=0.07, out=1, lse=1, ws=None, wsb=0)
    a.update(kw)
    return lib.mla_decode_varlen(a["q"], a["cu"], a["kv"], a["scale"], a["kind"], a["pt"], a["maxp"], a["lens"],
                                 a["batch"], a["tq"], a["mq"], a["heads"], a["page"], a["maxlen"], a["sf"],
                                 a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), mla.MLA_ERR_INVALID),
    (dict(q=None), mla.MLA_ERR_INVALID),
    (dict(tq=17), mla.MLA_ERR_INVALID),             # more tokens than batch * max_q_len
    (dict(tq=-1), mla.MLA_ERR_INVALID),
    (dict(mq=0), mla.MLA_ERR_INVALID),
    (dict(mq=9), mla.MLA_ERR_UNSUPPORTED),          # 144 folded rows
    (dict(kind=2), mla.MLA_ERR_INVALID),            # fp8 without scales
    (dict(page=96), mla.MLA_ERR_UNSUPPORTED),
    (dict(maxlen=3), mla.MLA_ERR_INVALID),
    (dict(ws=None, wsb=0), mla.MLA_ERR_WORKSPACE),
    (dict(tq=0), mla.MLA_OK),                       # nothing to do, no launch
])
def test_decode_varlen_argument_checks(lib, kw, code):
    assert _varlen_rc(lib, **kw) == code


def test_workspace_covers_varlen_decode(lib):
    # fewer tokens than batch * max_q_len still sizes the decode split
    ws = mla.mla_splitkv_workspace_size(4, 16, 4, 10, 65536, 0)
    assert ws >= mla.mla_decode_plan(4, 16, 4, 65536, 0, num_cus=256)[1]


@pytest.mark.parametrize("fn", ["mla_q_absorb", "mla_v_up"])
def test_absorb_argument_checks(lib, fn):
    f = getattr(lib, fn)
    assert f(1, 1, 1, -1, 16, None) == mla.MLA_ERR_INVALID
    assert f(1, 1, 1, 4, 0, None) == mla.MLA_ERR_INVALID
    assert f(None, 1, 1, 4, 16, None) == mla.MLA_ERR_INVALID
    assert f(1, None, 1, 4, 16, None) == mla.MLA_ERR_INVALID
    assert f(1, 1, None, 4, 16, None) == mla.MLA_ERR_INVALID
    assert f(None, None, None, 0, 16, None) == mla.MLA_OK        # nothing to do, no launch
    assert f(1, 1, 1, 1 << 30, 16, None) == mla.MLA_ERR_UNSUPPORTED


def test_noalloc_rejects_plans_beyond_its_scratch(lib):
    """A shape whose split-KV workspace exceeds the fixed 64 MiB scratch is refused before
    anything is enqueued (host-only: the plan is computed for 256 compute units)."""
    wsb = mla.mla_splitkv_workspace_size(4000, 16, 4, 16000, 262144, 0)
    assert wsb > mla.MLA_NOALLOC_SCRATCH_BYTES
    rc = lib.mla_decode_noalloc(1, 1, None, 0, 1, 4096, 1, 4000, 4, 16, 64, 262144, 0.07, 1, 1, None)
    assert rc == mla.MLA_ERR_SCRATCH
    # the scalar checks of mla_decode come first
    assert lib.mla_decode_noalloc(None, 1, None, 0, 1, 4096, 1, 4, 4, 16, 64, 262144, 0.07, 1, 1, None) == \
        mla.MLA_ERR_INVALID
    assert lib.mla_decode_noalloc(1, 1, None, 0, 1, 4096, 1, 4, 4, 16, 32, 262144, 0.07, 1, 1, None) == \
        mla.MLA_ERR_UNSUPPORTED
