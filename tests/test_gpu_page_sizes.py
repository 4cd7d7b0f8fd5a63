"""Page sizes other than 64 (GPU): a page of P = 64 k rows is, in memory, k consecutive
64-row sub-pages, which is how the kernels walk it.  Parity against the oracle (which
reads page_table[b][t / P], slot t % P), bitwise equality with the 64-row view of the
same memory, and the two-level layout of 128-row logical blocks inside 1536-row
physical blocks ([TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎", section
"Runtime：构建可扩展的推理引擎架构")."""
import numpy as np
import pytest
import torch

import mla_attention_paged_amd as mla
import oracle
import synth
from mla_gpu import assert_close, dev_bf16, host, run_decode, run_decode_varlen, run_prefill

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("page_size", [128, 256, 1536, 4096])
def test_decode_page_size_matches_oracle(page_size, kv_dtype):
    case = synth.make_decode_case(701, 3, 16, 4, seq_lens=[3100, 130, 2000], kv_dtype=kv_dtype,
                                  page_size=page_size)
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, f"decode page {page_size} {kv_dtype}")


def _as_64(cache):
    """The same memory as 64-row pages, with the page table expanded."""
    k = cache.page_size // 64
    pt = cache.page_table
    pt64 = (pt[:, :, None] * k + np.arange(k)[None, None, :]).reshape(pt.shape[0], -1).astype(np.int32)
    data = cache.data.reshape(cache.num_pages * k, 64, 576)
    scale = None if cache.scale is None else cache.scale.reshape(cache.num_pages * k, 64)
    return synth.PagedCache(cache.kv_dtype, data, scale, pt64, cache.kv_lens, cache.poison_page * k, 64)


@pytest.mark.parametrize("page_size", [128, 1536, 4096])
def test_decode_page_size_bitwise_equals_64_view(page_size):
    a = synth.make_decode_case(702, 2, 16, 2, seq_lens=[4000, 777], page_size=page_size)
    b = synth.DecodeCase(a.batch, a.heads, a.q_len, a.q, _as_64(a.cache), a.max_seq_len, a.softmax_scale)
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)


def test_decode_two_level_blocks():
    """128-row logical blocks placed in slots of 1536-row physical blocks: page_size 128,
    entry = physical block * 12 + slot."""
    rng = np.random.default_rng(703)
    case = synth.make_decode_case(703, 2, 16, 4, seq_lens=[2500, 1300], page_size=128)
    c = case.cache
    nphys = (c.num_pages + 11) // 12 + 1
    slots = rng.permutation(nphys * 12)[: c.num_pages]          # logical 128-page -> (block, slot)
    data = np.zeros((nphys * 12, 128, 576), dtype=c.data.dtype)
    data[slots] = c.data
    c.data = data
    c.page_table = slots[c.page_table].astype(np.int32)
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, "two-level blocks")


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("page_size", [1536, 4096])
def test_prefill_page_size_matches_oracle(page_size, kv_dtype):
    case = synth.make_prefill_case(704, 16, prefix_lens=[1600, 0, 100], new_lens=[30, 70, 5], kv_dtype=kv_dtype,
                                   page_size=page_size)
    out, lse = host(*run_prefill(case))
    ref_out, ref_lse = oracle.prefill(case)
    T = case.total_q()
    assert_close(out[:T], lse[:T], ref_out, ref_lse, f"prefill page {page_size} {kv_dtype}")


def test_decode_varlen_page_size_matches_oracle():
    case = synth.make_prefill_case(705, 16, prefix_lens=[300, 2000], new_lens=[3, 1], page_size=128)
    out, lse = host(*run_decode_varlen(case, max_q_len=4))
    ref_out, ref_lse = oracle.prefill(case)
    T = case.total_q()
    assert_close(out[:T], lse[:T], ref_out, ref_lse, "varlen page 128")


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("page_size", [128, 1536])
def test_append_page_size_bit_exact(page_size, kv_dtype):
    rng = np.random.default_rng(706)
    batch, entries = 2, 3
    num_pages = batch * entries + 1
    pt = rng.permutation(num_pages)[: batch * entries].reshape(batch, entries).astype(np.int32)
    if kv_dtype == "bf16":
        cache = rng.integers(0, 1 << 16, size=(num_pages, page_size, 576), dtype=np.uint16)
        scale = None
    else:
        cache = rng.integers(-127, 128, size=(num_pages, page_size, 576), dtype=np.int8)
        if kv_dtype == "fp8":
            cache = cache.view(np.uint8) & np.uint8(0xFE)   # no NaN codes
        scale = rng.random((num_pages, page_size), dtype=np.float32)
    start = np.array([page_size - 5, 3], np.int32)
    n = np.array([70, 9], np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    new = synth.bf16_bits(rng.standard_normal((int(cu[-1]), 576)).astype(np.float32))
    if kv_dtype == "bf16":
        kv = dev_bf16(cache)
        sc = None
        kind = mla.MLA_KV_BF16
    else:
        kv = torch.from_numpy(np.ascontiguousarray(cache)).cuda()
        sc = torch.from_numpy(scale).cuda()
        kind = mla.MLA_KV_INT8 if kv_dtype == "int8" else mla.MLA_KV_FP8
    mla.mla_kv_append(dev_bf16(new), torch.from_numpy(cu).cuda(), torch.from_numpy(start).cuda(), kv, sc, kind,
                      torch.from_numpy(pt).cuda(), entries, batch, int(cu[-1]), page_size)
    torch.cuda.synchronize()
    got = kv.view(torch.int16).cpu().numpy().view(np.uint16) if kv_dtype == "bf16" else kv.cpu().numpy()
    ref, ref_sc = oracle.kv_append(new, cu, start, cache, scale, kv_dtype, pt)
    assert np.array_equal(got, ref)
    if scale is not None:
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref_sc.view(np.uint32))
