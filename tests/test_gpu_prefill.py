"""Varlen prefill parity: the HIP path through the C ABI against the fp64 oracle (GPU)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from mla_gpu import assert_close, host, prefill_inputs, run_decode, run_prefill, sample_prefill_tokens

pytestmark = pytest.mark.gpu

SMALL = [
    # (seed, heads, prefix_lens, new_lens)
    (401, 16, [0], [1]),
    (402, 16, [100, 0, 64], [5, 70, 1]),
    (403, 16, [1000, 63, 64, 3], [17, 9, 65, 200]),
    (404, 8, [5, 300], [129, 2]),
    (405, 32, [640, 2], [33, 7]),
    (406, 128, [77, 10], [3, 2]),
    (407, 64, [0, 129], [4, 3]),
    (408, 16, [300, 0, 20], [0, 12, 0]),   # requests without new tokens
    (409, 3, [50], [40]),
]


@pytest.mark.parametrize("seed,heads,prefix,new", SMALL, ids=[str(s[0]) for s in SMALL])
def test_prefill_matches_oracle_small(seed, heads, prefix, new):
    case = synth.make_prefill_case(seed, heads, prefix_lens=prefix, new_lens=new)
    out, lse = host(*run_prefill(case))
    ref_out, ref_lse = oracle.prefill(case)
    T = case.total_q()
    assert_close(out[:T], lse[:T], ref_out, ref_lse, f"seed {seed}")


def test_prefill_ragged_batch():
    g = np.random.default_rng(9)
    prefix = g.integers(0, 2500, size=11)
    new = g.integers(1, 150, size=11)
    case = synth.make_prefill_case(410, 16, prefix_lens=prefix, new_lens=new)
    out, lse = host(*run_prefill(case))
    ref_out, ref_lse = oracle.prefill(case)
    assert_close(out, lse, ref_out, ref_lse, "ragged 11")


def test_prefill_many_requests():
    """600 requests (the work list orders and sums them in one workgroup): prefixes of
    0-300 rows, 0-6 new tokens each (empty requests included)."""
    g = np.random.default_rng(9)
    prefix = g.integers(0, 300, size=600)
    new = g.integers(0, 7, size=600)
    case = synth.make_prefill_case(421, 16, prefix_lens=prefix, new_lens=new)
    out, lse = host(*run_prefill(case))
    T = case.total_q()
    ref_out, ref_lse = oracle.prefill(case, nthreads=min(16, os.cpu_count() or 1))
    assert_close(out[:T], lse[:T], ref_out, ref_lse, "prefill 600 requests")


def test_prefill_rows_equal_decode_rows_on_gpu():
    """Prefill token j of a request equals decode with q_len=1 on its first P+j+1 rows."""
    case = synth.make_prefill_case(411, 16, prefix_lens=[200], new_lens=[5])
    po, pl = host(*run_prefill(case))
    ref_out, ref_lse = oracle.prefill(case)
    assert_close(po, pl, ref_out, ref_lse, "prefill")
    for j in range(5):
        d = synth.DecodeCase(1, 16, 1, case.q[j:j + 1].copy(),
                             synth.PagedCache("bf16", case.cache.data, None, case.cache.page_table,
                                              np.array([200 + j + 1], np.int32), case.cache.poison_page),
                             max_seq_len=205)
        do, dl = host(*run_decode(d))
        assert_close(do[0:1], dl[0:1], ref_out[j:j + 1], ref_lse[j:j + 1], f"decode row {j}")


def test_prefill_deterministic():
    case = synth.make_prefill_case(412, 16, prefix_lens=[900, 50, 2000], new_lens=[40, 300, 9])
    d = prefill_inputs(case)
    o1, l1 = run_prefill(case, d)
    o2, l2 = run_prefill(case, d)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_prefill_nan_poison_has_no_effect():
    a = synth.make_prefill_case(413, 16, prefix_lens=[10, 100], new_lens=[3, 30])
    b = synth.make_prefill_case(413, 16, prefix_lens=[10, 100], new_lens=[3, 30], poison=synth.POISON_NAN)
    oa, la = run_prefill(a)
    ob, lb = run_prefill(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)


def test_prefill_workload3_sampled():
    """The full 8-request prefill as benchmarked; the oracle evaluates the first and last
    new token of every request and one token from a seeded 1/32 of the work tiles (4
    tokens x 16 heads each), all heads."""
    case = synth.make_workload(3)
    out, lse = host(*run_prefill(case))
    toks = sample_prefill_tokens(case, 64 // case.heads, seed=30)
    assert len(toks) > 60
    ref_out, ref_lse = oracle.prefill(case, tokens=toks, nthreads=min(16, os.cpu_count() or 1))
    errs = assert_close(out[toks], lse[toks], ref_out, ref_lse, f"{case.name} ({len(toks)} tokens)")
    print("workload3 sampled: max abs err %.3g, lse err %.3g, rel frob %.3g" % errs)


@pytest.mark.parametrize("seed,heads,prefix,new", [(420, 16, [100, 0, 64], [5, 70, 1]),
                                                   (421, 128, [77, 10], [3, 2]),
                                                   (422, 16, [1000, 63], [17, 9])])
def test_prefill_int8_matches_oracle(seed, heads, prefix, new):
    case = synth.make_prefill_case(seed, heads, prefix_lens=prefix, new_lens=new, kv_dtype="int8")
    out, lse = host(*run_prefill(case))
    ref_out, ref_lse = oracle.prefill(case)
    T = case.total_q()
    assert_close(out[:T], lse[:T], ref_out, ref_lse, f"int8 seed {seed}")


@pytest.mark.parametrize("seed,heads,prefix,new", [(430, 16, [100, 0, 64], [5, 70, 1]),
                                                   (431, 128, [77, 10], [3, 2]),
                                                   (432, 16, [1000, 63], [17, 9])])
def test_prefill_fp8_matches_oracle(seed, heads, prefix, new):
    case = synth.make_prefill_case(seed, heads, prefix_lens=prefix, new_lens=new, kv_dtype="fp8")
    out, lse = host(*run_prefill(case))
    ref_out, ref_lse = oracle.prefill(case)
    T = case.total_q()
    assert_close(out[:T], lse[:T], ref_out, ref_lse, f"fp8 seed {seed}")
