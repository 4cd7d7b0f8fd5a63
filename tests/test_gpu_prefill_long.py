"""Prefill parity at long prefixes (GPU): sampled oracle parity on the 8-request prefill
workload's shape for the INT8 and FP8 caches, and bit-exact gather, causal-mask and
page-placement checks on prefixes longer than the kernels' 256-page (16,384-row) window
of staged page ids, so that the window restart runs under every check."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from mla_gpu import assert_close, bits, host, permute_pages, prefill_inputs, run_prefill, sample_prefill_tokens

pytestmark = pytest.mark.gpu

NT = min(16, os.cpu_count() or 1)
WIN = 16384                      # rows per window of staged page ids in the prefill kernels
BF16_64 = int(synth.bf16_bits(np.array([64.0], np.float32))[0])
BF16_32 = int(synth.bf16_bits(np.array([32.0], np.float32))[0])
E4M3_128 = 0x70                  # E4M3: exponent field 14 (bias 7), mantissa 0 -> 128
NEEDLE_SCALE = np.float32(0.25)  # a power of two: the needle's dequantised values are exact in bf16


def _tok_per_tile(heads):
    return 1 if heads >= 64 else 64 // heads


def _workload3(kv_dtype):
    base = synth.make_workload(3)
    if kv_dtype == "bf16":
        return base
    return synth.make_prefill_case(4, base.heads, prefix_lens=base.prefix_lens,
                                   new_lens=np.diff(base.cu_seqlens_q), kv_dtype=kv_dtype,
                                   name=f"{base.name}_{kv_dtype}")


@pytest.mark.parametrize("kv_dtype", ["int8", "fp8"])
def test_prefill_codes_workload3_sampled(kv_dtype):
    """The 8-request prefill (prefixes 23K-96K rows, 8,629 new tokens, 16 heads) with an
    INT8 / FP8 cache, as benchmarked; the oracle evaluates the first and last new token of
    each request and one token from a seeded 1/32 of the work tiles, all heads."""
    case = _workload3(kv_dtype)
    out, lse = host(*run_prefill(case))
    toks = sample_prefill_tokens(case, _tok_per_tile(case.heads), seed=31)
    ref_out, ref_lse = oracle.prefill(case, tokens=toks, nthreads=NT)
    assert_close(out[toks], lse[toks], ref_out, ref_lse, f"{case.name} ({len(toks)} tokens)")


def _set_needle(case, b, pos, js):
    """Row `pos` of request b gets the needle: value 32 at column js[h] for every head h
    (bf16: the value itself; INT8: code 127, FP8: code 128, both with row scale 1/4)."""
    c = case.cache
    page, slot = c.page_table[b, pos // c.page_size], pos % c.page_size
    for j in js:
        if c.kv_dtype == "bf16":
            c.data[page, slot, j] = BF16_32
        elif c.kv_dtype == "int8":
            c.data[page, slot, j] = 127
        else:
            c.data[page, slot, j] = E4M3_128
    if c.kv_dtype != "bf16":
        c.scale[page, slot] = NEEDLE_SCALE


def _row_value_bits(case, b, pos):
    """bf16 bits of the dequantised value columns of row `pos` of request b (exact: bf16
    rows as stored; codes times the power-of-two scale 1/4 of a needle row)."""
    c = case.cache
    page, slot = c.page_table[b, pos // c.page_size], pos % c.page_size
    if c.kv_dtype == "bf16":
        return c.data[page, slot, :512].copy()
    assert c.scale[page, slot] == NEEDLE_SCALE
    codes = c.data[page, slot, :512]
    if c.kv_dtype == "int8":
        vals = codes.astype(np.float32) * NEEDLE_SCALE
    else:
        vals = np.array([oracle.e4m3_value(int(x)) for x in codes], np.float32) * NEEDLE_SCALE
    return synth.bf16_bits(vals)


def _needle_queries(case, b, js):
    cu = case.cu_seqlens_q
    for t in range(int(cu[b]), int(cu[b + 1])):
        for h, j in enumerate(js):
            q = np.zeros(576, np.uint16)
            q[j] = BF16_64
            case.q[t, h] = q


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
def test_prefill_needle_long_bit_exact(kv_dtype):
    """q = 64 e_j and one prefix row with 32 at column j (per head): that row's score leads
    every other by > 100 (natural units), every other weight underflows to 0 in fp32 and
    each new token's output must be the needle row's value columns bit for bit.  Needles
    sit on page edges and on both sides of the 16,384-row window edge."""
    positions = [0, 63, 64, WIN - 1, WIN, WIN + 63, WIN + 64, 16900]
    prefix = [16901 + 7 * i for i in range(len(positions))]
    new = [9, 1, 4, 13, 5, 8, 3, 6]
    case = synth.make_prefill_case(601, 16, prefix_lens=prefix, new_lens=new, kv_dtype=kv_dtype)
    g = np.random.default_rng(61)
    js_all = g.integers(0, 512, size=(len(positions), 16))
    for b, pos in enumerate(positions):
        _set_needle(case, b, pos, js_all[b])
        _needle_queries(case, b, js_all[b])
    out, _ = run_prefill(case)
    got = bits(out)
    cu = case.cu_seqlens_q
    for b, pos in enumerate(positions):
        want = _row_value_bits(case, b, pos)
        for t in range(int(cu[b]), int(cu[b + 1])):
            for h in range(16):
                assert np.array_equal(got[t, h], want), f"{kv_dtype} needle at {pos} (request {b}), token {t}, head {h}"


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_prefill_causal_needle_long(kv_dtype):
    """A needle in the new tokens' own rows, at row P + k of a request with prefix P past the
    window edge: new tokens i >= k see it (bit-exact), tokens i < k must not (oracle
    parity, and the oracle excludes it).  k and P vary so that the needle falls at
    different places of the diagonal tiles (first / last token of a 4-token work tile,
    first / last row of a 32-row cache tile, the window's first row)."""
    cases = [(WIN, 0), (WIN + 5, 3), (WIN + 28, 4), (WIN + 31, 7), (17000, 11), (WIN + 60, 12)]
    n = 14
    prefix = [p for p, _ in cases]
    case = synth.make_prefill_case(602, 16, prefix_lens=prefix, new_lens=[n] * len(cases), kv_dtype=kv_dtype)
    g = np.random.default_rng(62)
    js_all = g.integers(0, 512, size=(len(cases), 16))
    for b, (P, k) in enumerate(cases):
        _set_needle(case, b, P + k, js_all[b])
        _needle_queries(case, b, js_all[b])
    out, lse = run_prefill(case)
    got = bits(out)
    early = []
    for b, (P, k) in enumerate(cases):
        want = _row_value_bits(case, b, P + k)
        t0 = int(case.cu_seqlens_q[b])
        for i in range(k, n):
            for h in range(16):
                assert np.array_equal(got[t0 + i, h], want), f"{kv_dtype} causal needle P={P} k={k}: token {i} head {h}"
        early += [t0 + i for i in range(k)]
    ref_out, ref_lse = oracle.prefill(case, tokens=early, nthreads=NT)
    o, l_ = host(out, lse)
    assert_close(o[early], l_[early], ref_out, ref_lse, f"{kv_dtype} tokens before the causal needle")


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
def test_prefill_page_permutation_long_bitwise(kv_dtype):
    """The same logical rows at other physical pages give the same bits (prefixes past the
    window edge, ragged new-token counts)."""
    kw = dict(prefix_lens=[17000, 33000, 40], new_lens=[50, 7, 300], kv_dtype=kv_dtype)
    a = synth.make_prefill_case(603, 16, **kw)
    b = synth.make_prefill_case(603, 16, **kw)
    permute_pages(b.cache, 63)
    oa, la = run_prefill(a)
    ob, lb = run_prefill(b)
    torch.cuda.synchronize()
    assert np.array_equal(bits(oa), bits(ob)) and torch.equal(la, lb)


def test_prefill_long_matches_oracle_all_tokens():
    """Every new token of two requests whose prefixes cross the window edge (one of them
    twice), all heads, against the oracle."""
    case = synth.make_prefill_case(604, 16, prefix_lens=[WIN + 3, 2 * WIN + 100], new_lens=[37, 22])
    out, lse = host(*run_prefill(case))
    ref_out, ref_lse = oracle.prefill(case, nthreads=NT)
    assert_close(out, lse, ref_out, ref_lse, "prefixes across the window edge")


def test_prefill_fp8_nan_code_tail_has_no_effect():
    """FP8 prefill: rows past each request's end hold the E4M3 NaN code 0x7F with a NaN
    scale; the output must equal the run with finite poison bit for bit."""
    kw = dict(prefix_lens=[WIN + 5, 300], new_lens=[33, 7], kv_dtype="fp8")
    a = synth.make_prefill_case(605, 16, **kw)
    b = synth.make_prefill_case(605, 16, **kw)
    c = b.cache
    for bb, L in enumerate(c.kv_lens):
        n = (int(L) + 63) // 64
        c.data[c.page_table[bb, n - 1], int(L) - 64 * (n - 1):] = 0x7F
        c.scale[c.page_table[bb, n - 1], int(L) - 64 * (n - 1):] = np.float32("nan")
    oa, la = run_prefill(a)
    ob, lb = run_prefill(b)
    torch.cuda.synchronize()
    assert np.array_equal(bits(oa), bits(ob)) and torch.equal(la, lb)
    assert torch.isfinite(ob.float()).all()


def test_prefill_million_row_prefix_sampled():
    """One request with a 1,048,571-row cached prefix (64 windows of staged page ids, a
    ragged last page) and 1,500 new tokens, beside a short one.  The oracle checks the long
    request's first and last new token and the short one's last, all heads: the first and
    last work tiles of the long request walk every window."""
    case = synth.make_prefill_case(532, 16, prefix_lens=[(1 << 20) - 5, 300], new_lens=[1500, 37])
    out, lse = host(*run_prefill(case))
    toks = [0, 1499, 1536]
    ref_out, ref_lse = oracle.prefill(case, tokens=toks, nthreads=NT)
    errs = assert_close(out[toks], lse[toks], ref_out, ref_lse, "1M prefix")
    print("million-row prefix: max abs err %.3g, lse err %.3g, rel frob %.3g" % errs)
