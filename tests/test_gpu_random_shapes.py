"""Seeded random shapes against the oracle (GPU): batch, heads, drafts, cache format,
page size and lengths drawn at random (small enough for the oracle), for the decode,
the ragged decode and the prefill.  Each case prints its draw so that a failure names
it."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from mla_gpu import assert_close, host, run_decode, run_decode_varlen, run_prefill

pytestmark = pytest.mark.gpu

NT = min(16, os.cpu_count() or 1)
HEADS = [1, 2, 3, 4, 8, 16, 20, 32, 64, 128]
PAGE_SIZES = [64, 64, 64, 128, 256, 1536]
KINDS = ["bf16", "bf16", "int8", "fp8"]


def _cus_env(n):
    old = os.environ.get("MLA_NUM_CUS")
    if n:
        os.environ["MLA_NUM_CUS"] = str(n)
    return old


def _restore(old):
    if old is None:
        os.environ.pop("MLA_NUM_CUS", None)
    else:
        os.environ["MLA_NUM_CUS"] = old


@pytest.mark.parametrize("seed", range(24))
def test_decode_random_shape(seed):
    rng = np.random.default_rng(9000 + seed)
    heads = int(rng.choice(HEADS))
    q_len = int(rng.integers(1, 5)) if heads <= 32 else 1
    batch = int(rng.integers(1, 13))
    page = int(rng.choice(PAGE_SIZES))
    kind = str(rng.choice(KINDS))
    lens = rng.integers(q_len, 6000, size=batch)
    cus = int(rng.choice([0, 0, 1, 5, 37, 300]))
    draw = f"seed {seed}: batch {batch} heads {heads} q_len {q_len} page {page} {kind} cus {cus} lens {lens.tolist()}"
    print(draw, flush=True)
    case = synth.make_decode_case(9000 + seed, batch, heads, q_len, seq_lens=lens, kv_dtype=kind, page_size=page)
    old = _cus_env(cus)
    try:
        out, lse = run_decode(case)
        torch.cuda.synchronize()
    finally:
        _restore(old)
    ref_out, ref_lse = oracle.decode(case, nthreads=NT)
    assert_close(*host(out, lse), ref_out, ref_lse, draw)


@pytest.mark.parametrize("seed", range(8))
def test_decode_varlen_random_shape(seed):
    rng = np.random.default_rng(9100 + seed)
    heads = int(rng.choice([4, 8, 16, 32]))
    batch = int(rng.integers(1, 10))
    kind = str(rng.choice(KINDS))
    new = rng.integers(1, 5, size=batch)
    prefix = rng.integers(0, 5000, size=batch)
    draw = f"seed {seed}: batch {batch} heads {heads} {kind} prefix {prefix.tolist()} drafts {new.tolist()}"
    print(draw, flush=True)
    case = synth.make_prefill_case(9100 + seed, heads, prefix_lens=prefix, new_lens=new, kv_dtype=kind)
    out, lse = run_decode_varlen(case)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.prefill(case, nthreads=NT)
    assert_close(*host(out, lse), ref_out, ref_lse, draw)


@pytest.mark.parametrize("seed", range(12))
def test_prefill_random_shape(seed):
    rng = np.random.default_rng(9200 + seed)
    heads = int(rng.choice([1, 2, 8, 16, 32, 64]))
    batch = int(rng.integers(1, 7))
    page = int(rng.choice(PAGE_SIZES))
    kind = str(rng.choice(KINDS))
    new = rng.integers(0, 90, size=batch)
    new[rng.integers(0, batch)] = max(1, int(new.max()))
    prefix = rng.integers(0, 3000, size=batch)
    draw = f"seed {seed}: batch {batch} heads {heads} page {page} {kind} prefix {prefix.tolist()} new {new.tolist()}"
    print(draw, flush=True)
    case = synth.make_prefill_case(9200 + seed, heads, prefix_lens=prefix, new_lens=new, kv_dtype=kind,
                                   page_size=page)
    out, lse = run_prefill(case)
    torch.cuda.synchronize()
    T = case.total_q()
    ref_out, ref_lse = oracle.prefill(case, nthreads=NT)
    assert_close(*host(out[:T], lse[:T]), ref_out, ref_lse, draw)
