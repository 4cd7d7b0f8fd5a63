"""KV append parity: the HIP kernel through the C ABI against the oracle, bit-exact (GPU).

bf16 rows must land unchanged and INT8 / FP8 codes and scales must equal the
oracle's to the bit; nothing outside the written slots may change."""
import numpy as np
import pytest
import torch

import mla_attention_paged_amd as mla
import oracle
import synth
from mla_gpu import assert_close, dev_bf16, host, run_decode

pytestmark = pytest.mark.gpu


def _fresh_cache(rng, kv_dtype, num_pages):
    if kv_dtype == "bf16":
        return rng.integers(0, 1 << 16, size=(num_pages, 64, 576), dtype=np.uint16), None
    if kv_dtype == "fp8":
        codes = rng.integers(0, 256, size=(num_pages, 64, 576), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x7E
        return codes, (rng.random((num_pages, 64), dtype=np.float32) + np.float32(0.5))
    return (rng.integers(-127, 128, size=(num_pages, 64, 576), dtype=np.int8),
            (rng.random((num_pages, 64), dtype=np.float32) + np.float32(0.5)))


def run_append(new_bits, cu, start, cache, scale, kv_dtype, pt):
    """Append on the GPU; returns host copies of the cache (and scales)."""
    if kv_dtype == "bf16":
        kv = dev_bf16(cache)
        sc = None
        kind = mla.MLA_KV_BF16
    else:
        kv = torch.from_numpy(np.ascontiguousarray(cache)).cuda()
        sc = torch.from_numpy(np.ascontiguousarray(scale)).cuda()
        kind = mla.MLA_KV_INT8 if kv_dtype == "int8" else mla.MLA_KV_FP8
    new = dev_bf16(np.ascontiguousarray(new_bits).reshape(-1, 576))
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    st_d = torch.from_numpy(np.asarray(start, np.int32)).cuda()
    pt_d = torch.from_numpy(np.ascontiguousarray(pt, dtype=np.int32)).cuda()
    mla.mla_kv_append(new, cu_d, st_d, kv, sc, kind, pt_d, pt.shape[1], len(start), int(cu[-1]), 64)
    torch.cuda.synchronize()
    if kv_dtype == "bf16":
        return kv.view(torch.int16).cpu().numpy().view(np.uint16), None
    return kv.cpu().numpy(), sc.cpu().numpy()


def _check(new_bits, cu, start, cache, scale, kv_dtype, pt):
    got, got_sc = run_append(new_bits, cu, start, cache, scale, kv_dtype, pt)
    ref, ref_sc = oracle.kv_append(new_bits, cu, start, cache, scale, kv_dtype, pt)
    assert np.array_equal(got, ref)
    if kv_dtype != "bf16":
        assert np.array_equal(got_sc.view(np.uint32), ref_sc.view(np.uint32))


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
def test_append_ragged_matches_oracle(kv_dtype):
    rng = np.random.default_rng(31)
    batch, max_pages = 4, 6
    num_pages = batch * max_pages + 1
    pt = rng.permutation(num_pages - 1)[: batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    cache, scale = _fresh_cache(rng, kv_dtype, num_pages)
    start = np.array([0, 63, 130, 64], np.int32)
    n = np.array([5, 70, 3, 0], np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    new = synth.bf16_bits(rng.standard_normal((int(cu[-1]), 576)).astype(np.float32) * np.float32(3.0))
    _check(new, cu, start, cache, scale, kv_dtype, pt)


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
def test_append_many_requests_with_empty_ones(kv_dtype):
    """150 requests (the row-to-request lookup reads 64 request offsets per round trip),
    runs of empty requests among them, also at the 64-request boundaries."""
    rng = np.random.default_rng(39)
    batch, max_pages = 150, 2
    num_pages = batch * max_pages
    pt = rng.permutation(num_pages).reshape(batch, max_pages).astype(np.int32)
    cache, scale = _fresh_cache(rng, kv_dtype, num_pages)
    n = rng.integers(0, 4, size=batch).astype(np.int32)
    n[[0, 5, 6, 7, 62, 63, 64, 65, 127, 128, 149]] = 0
    n[[1, 66, 129]] = 9
    start = rng.integers(0, max_pages * 64 - 9, size=batch).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    new = synth.bf16_bits(rng.standard_normal((int(cu[-1]), 576)).astype(np.float32))
    _check(new, cu, start, cache, scale, kv_dtype, pt)


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
def test_append_edge_rows(kv_dtype):
    """Rows past the page table are dropped; zero rows, ties and huge / tiny magnitudes."""
    rng = np.random.default_rng(32)
    batch, max_pages = 2, 3
    num_pages = batch * max_pages
    pt = np.arange(num_pages, dtype=np.int32)[::-1].reshape(batch, max_pages).copy()
    cache, scale = _fresh_cache(rng, kv_dtype, num_pages)
    start = np.array([max_pages * 64 - 3, 0], np.int32)   # request 0 spills 4 rows past its table
    n = np.array([7, 6], np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    x = rng.standard_normal((13, 576)).astype(np.float32)
    x[7] = 0.0                                              # all-zero row
    x[8, :4] = [127.0, 2.5, -3.5, 0.5]                      # ties at scale 1
    x[8, 4:] = 0.0
    x[9] *= np.float32(1e30)
    x[10] *= np.float32(1e-30)
    x[11, 5] = np.float32(-1e4)                             # one dominant value
    new = synth.bf16_bits(x)
    _check(new, cu, start, cache, scale, kv_dtype, pt)


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
def test_append_prefill_workload_tokens(kv_dtype):
    """The long-prefix prefill's 8,629 new tokens, appended at their prefix positions."""
    case = synth.make_workload(3)
    rng = np.random.default_rng(33)
    pt = case.cache.page_table
    num_pages = int(pt.max()) + 1
    cache, scale = _fresh_cache(rng, kv_dtype, num_pages)
    cu = case.cu_seqlens_q.astype(np.int32)
    start = case.prefix_lens.astype(np.int32)
    new = synth.bf16_bits(rng.standard_normal((int(cu[-1]), 576)).astype(np.float32))
    _check(new, cu, start, cache, scale, kv_dtype, pt)


def _logical_rows(cache):
    rows = []
    for b in range(len(cache.kv_lens)):
        for t in range(int(cache.kv_lens[b])):
            rows.append(cache.data[cache.page_table[b, t // 64], t % 64])
    return np.stack(rows)


def test_append_then_decode_bf16_bitwise():
    """A cache rebuilt by appending every row decodes exactly like the original."""
    case = synth.make_decode_case(541, batch=3, heads=16, q_len=2, seq_lens=[300, 65, 129])
    c = case.cache
    rows = _logical_rows(c)
    cu = np.concatenate([[0], np.cumsum(c.kv_lens)]).astype(np.int32)
    rebuilt, _ = run_append(rows, cu, np.zeros(3, np.int32), np.zeros_like(c.data), None, "bf16", c.page_table)
    case2 = synth.DecodeCase(case.batch, case.heads, case.q_len, case.q,
                             synth.PagedCache("bf16", rebuilt, None, c.page_table, c.kv_lens, c.poison_page),
                             max_seq_len=case.max_seq_len)
    o1, l1 = run_decode(case)
    o2, l2 = run_decode(case2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_append_then_decode_int8():
    """Quantise a bf16 cache with the append kernel, then decode it: matches the oracle
    on the oracle-quantised cache (which is bit-identical)."""
    case = synth.make_decode_case(542, batch=2, heads=16, q_len=4, seq_lens=[700, 257])
    c = case.cache
    rows = _logical_rows(c)
    cu = np.concatenate([[0], np.cumsum(c.kv_lens)]).astype(np.int32)
    num_pages = c.data.shape[0]
    codes0 = np.zeros((num_pages, 64, 576), np.int8)
    scale0 = np.ones((num_pages, 64), np.float32)
    got, got_sc = run_append(rows, cu, np.zeros(2, np.int32), codes0, scale0, "int8", c.page_table)
    ref, ref_sc = oracle.kv_append(rows, cu, np.zeros(2, np.int32), codes0, scale0, "int8", c.page_table)
    assert np.array_equal(got, ref) and np.array_equal(got_sc.view(np.uint32), ref_sc.view(np.uint32))
    case8 = synth.DecodeCase(case.batch, case.heads, case.q_len, case.q,
                             synth.PagedCache("int8", got, got_sc, c.page_table, c.kv_lens, c.poison_page),
                             max_seq_len=case.max_seq_len)
    out, lse = host(*run_decode(case8))
    ref_out, ref_lse = oracle.decode(case8)
    assert_close(out, lse, ref_out, ref_lse, "append-quantised int8 decode")


def test_append_fp8_rounding_edges():
    """max|x| = 448 makes the scale exactly 1, so the codes are the E4M3 rounding of the
    inputs themselves: ties to even in the normal and subnormal ranges, values that round
    up into the next binade, the smallest subnormals, signed zeros."""
    pt = np.arange(2, dtype=np.int32).reshape(1, 2)
    cache, scale = _fresh_cache(np.random.default_rng(34), "fp8", 2)
    x = np.zeros((3, 576), np.float32)
    vals = [448.0, 17.0, 19.0, -17.0, -19.0, 2.0 ** -10, 3 * 2.0 ** -10, 5 * 2.0 ** -10, -3 * 2.0 ** -10,
            2.0 ** -6 - 2.0 ** -10, 31.0, 30.0, 1.0625, 1.1875, 240.0, 416.0, 432.0, -0.0, 2.0 ** -9,
            0.9375 * 2.0 ** -6, 15.5, 0.09375]
    x[0, :len(vals)] = vals
    x[1] = x[0] * np.float32(-1.0)
    x[2, 0] = 448.0
    x[2, 1:] = np.random.default_rng(35).uniform(-448, 448, 575).astype(np.float32)
    new = synth.bf16_bits(x)
    assert np.array_equal(synth.bf16_to_f32(new)[0, :len(vals)], x[0, :len(vals)])   # exact inputs
    cu = np.array([0, 3], np.int32)
    _check(new, cu, np.array([5], np.int32), cache, scale, "fp8", pt)


def _near_boundary_rows(kv_dtype, seed, n_scales=300):
    """Rows of bf16 values whose fp32 quotient x / scale lies on or within 4 ulps of a
    rounding boundary of the code (a half-integer for INT8, a midpoint between adjacent
    E4M3 values for FP8), each row led by its max magnitude A so that its scale is
    fp32(A / 127) or fp32(A / 448).  Power-of-two scales (A = 127 or 448) add exact
    ties.  Returns (bf16 bits [rows, 576], number of near-boundary values)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    m = np.float32(127.0 if kv_dtype == "int8" else 448.0)
    rng = np.random.default_rng(seed)
    amaxes = list(rng.choice(vals[(vals > 0.01) & (vals < 1000)], n_scales, replace=False)) + [m, m * 2, m / 4]
    rows, count = [], 0
    for a in amaxes:
        scale = np.float32(np.float32(a) / m)
        x = vals[np.abs(vals) <= a]
        q = np.abs((x / scale).astype(np.float32)).astype(np.float64)
        ulp = np.spacing(q.astype(np.float32)).astype(np.float64)
        if kv_dtype == "int8":
            d = np.abs(q - np.floor(q) - 0.5)
        else:
            with np.errstate(divide="ignore"):
                e = np.maximum(np.floor(np.log2(np.where(q > 0, q, 1.0))), -6)
            grid = 2.0 ** (e - 3)
            d = np.abs(q / grid - np.floor(q / grid) - 0.5) * grid
        near = x[(d <= 4 * ulp) & (q > 0)][:575]
        if len(near) == 0:
            continue
        row = np.zeros(576, np.float32)
        row[0] = a
        row[1:1 + len(near)] = near
        rows.append(row)
        count += len(near)
    return synth.bf16_bits(np.stack(rows)), count


@pytest.mark.parametrize("kv_dtype", ["int8", "fp8"])
def test_append_codes_near_rounding_boundaries(kv_dtype):
    """Quotients on or next to a rounding boundary of the code must round exactly as the
    correctly rounded fp32 division x / scale does (ties to even)."""
    new, count = _near_boundary_rows(kv_dtype, 36 if kv_dtype == "int8" else 37)
    assert count > (1000 if kv_dtype == "int8" else 5000)
    rows = new.shape[0]
    pages = (rows + 63) // 64
    pt = np.arange(pages, dtype=np.int32).reshape(1, pages)
    cache, scale = _fresh_cache(np.random.default_rng(38), kv_dtype, pages)
    _check(new, np.array([0, rows], np.int32), np.array([0], np.int32), cache, scale, kv_dtype, pt)


def test_append_then_decode_fp8():
    """Quantise a bf16 cache to FP8 with the append kernel, then decode it: matches the
    oracle on the oracle-quantised cache (which is bit-identical)."""
    case = synth.make_decode_case(543, batch=2, heads=16, q_len=4, seq_lens=[700, 257])
    c = case.cache
    rows = _logical_rows(c)
    cu = np.concatenate([[0], np.cumsum(c.kv_lens)]).astype(np.int32)
    num_pages = c.data.shape[0]
    codes0 = np.zeros((num_pages, 64, 576), np.uint8)
    scale0 = np.ones((num_pages, 64), np.float32)
    got, got_sc = run_append(rows, cu, np.zeros(2, np.int32), codes0, scale0, "fp8", c.page_table)
    ref, ref_sc = oracle.kv_append(rows, cu, np.zeros(2, np.int32), codes0, scale0, "fp8", c.page_table)
    assert np.array_equal(got, ref) and np.array_equal(got_sc.view(np.uint32), ref_sc.view(np.uint32))
    case8 = synth.DecodeCase(case.batch, case.heads, case.q_len, case.q,
                             synth.PagedCache("fp8", got, got_sc, c.page_table, c.kv_lens, c.poison_page),
                             max_seq_len=case.max_seq_len)
    out, lse = host(*run_decode(case8))
    ref_out, ref_lse = oracle.decode(case8)
    assert_close(out, lse, ref_out, ref_lse, "append-quantised fp8 decode")
