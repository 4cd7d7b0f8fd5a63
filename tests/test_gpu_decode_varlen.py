"""Decode with a different number of query tokens per request (speculative decoding
with a variable number of drafts) through mla_decode_varlen, against the oracle (GPU).

A ragged decode case is built as a prefill-shaped case whose prefix is L_b - n_b: the
oracle's definition is the same (token i of request b sees rows 0 .. L_b - n_b + i)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from mla_gpu import assert_close, decode_inputs, host, run_decode, run_decode_varlen

pytestmark = pytest.mark.gpu

CASES = [
    # (seed, heads, seq_lens, q_lens)
    (601, 16, [300, 70, 1000, 5], [1, 4, 2, 3]),
    (602, 16, [129, 64, 2000], [8, 0, 5]),            # 128 folded rows (two blocks); an empty request
    (603, 32, [65, 640, 77, 3000, 12], [2, 4, 1, 3, 4]),
    (604, 128, [700, 90], [1, 1]),
    (605, 16, [9], [8]),                              # every row is a draft
]


def _case(seed, heads, seq_lens, q_lens, kv_dtype="bf16"):
    seq_lens = np.asarray(seq_lens)
    q_lens = np.asarray(q_lens)
    return synth.make_prefill_case(seed, heads, prefix_lens=seq_lens - q_lens, new_lens=q_lens, kv_dtype=kv_dtype)


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("seed,heads,seq_lens,q_lens", CASES, ids=[str(c[0]) for c in CASES])
def test_decode_varlen_matches_oracle(seed, heads, seq_lens, q_lens, kv_dtype):
    case = _case(seed, heads, seq_lens, q_lens, kv_dtype)
    mq = max(q_lens)
    out, lse = host(*run_decode_varlen(case, max_q_len=mq))
    ref_out, ref_lse = oracle.prefill(case)
    T = case.total_q()
    assert_close(out[:T], lse[:T], ref_out, ref_lse, f"varlen {kv_dtype} seed {seed}")


def test_decode_varlen_uniform_equals_decode_bitwise():
    """Equal counts through the ragged entry point give the uniform kernel's bits."""
    d = synth.make_decode_case(606, 3, 16, 4, seq_lens=[900, 333, 4000])
    o1, l1 = run_decode(d)
    p = synth.PrefillCase(d.heads, d.q, d.q_start(), (d.seq_lens - d.q_len).astype(np.int32), d.cache,
                          d.max_seq_len, d.softmax_scale)
    o2, l2 = run_decode_varlen(p, max_q_len=4)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("cus", [1, 7, 256])
def test_decode_varlen_split_plans_agree(cus):
    case = _case(607, 16, [1500, 64, 777, 2], [3, 1, 4, 2])
    old = os.environ.get("MLA_NUM_CUS")
    os.environ["MLA_NUM_CUS"] = str(cus)
    try:
        out, lse = host(*run_decode_varlen(case, max_q_len=4))
    finally:
        if old is None:
            os.environ.pop("MLA_NUM_CUS", None)
        else:
            os.environ["MLA_NUM_CUS"] = old
    ref_out, ref_lse = oracle.prefill(case)
    T = case.total_q()
    assert_close(out[:T], lse[:T], ref_out, ref_lse, f"varlen cus {cus}")


def test_decode_varlen_long_sampled():
    """Four 64K-row requests with 1..4 drafts; the oracle evaluates every request's first and last token."""
    case = _case(608, 16, [65536] * 4, [1, 2, 3, 4])
    out, lse = host(*run_decode_varlen(case, max_q_len=4))
    cu = case.cu_seqlens_q
    toks = sorted({int(cu[b]) for b in range(4)} | {int(cu[b + 1]) - 1 for b in range(4)})
    ref_out, ref_lse = oracle.prefill(case, tokens=toks, nthreads=min(16, os.cpu_count() or 1))
    assert_close(out[toks], lse[toks], ref_out, ref_lse, "varlen 64K")


def test_decode_varlen_no_tokens():
    case = _case(609, 16, [100, 50], [0, 0])
    out, lse = run_decode_varlen(case, max_q_len=2)   # enqueues nothing, must not fail
    torch.cuda.synchronize()


def test_decode_varlen_more_requests_than_the_offset_cache():
    """600 requests with 0-4 drafts each: query offsets past the 512 the kernels cache in
    LDS come from memory; empty requests in between."""
    g = np.random.default_rng(8)
    q_lens = g.integers(0, 5, size=600)
    seq_lens = q_lens + g.integers(0, 300, size=600)
    seq_lens = np.maximum(seq_lens, 1)
    case = _case(612, 16, seq_lens, q_lens)
    out, lse = run_decode_varlen(case)
    T = case.total_q()
    ref_out, ref_lse = oracle.prefill(case, nthreads=min(16, os.cpu_count() or 1))
    o, l_ = host(out, lse)
    assert_close(o[:T], l_[:T], ref_out, ref_lse, "varlen 600 requests")
