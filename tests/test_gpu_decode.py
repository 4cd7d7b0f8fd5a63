"""Decode parity: the HIP path through the C ABI against the fp64 oracle (GPU)."""
import os

import numpy as np
import pytest
import torch

import mla_attention_paged_amd as mla
import oracle
import synth
from mla_gpu import assert_close, decode_inputs, host, run_decode

pytestmark = pytest.mark.gpu

BF16_ONE = 0x3F80


def _put_row(case, b, t, values_bits):
    c = case.cache
    page = c.page_table[b, t // 64]
    c.data[page, t % 64] = values_bits


def _row_bits(case, b, t):
    c = case.cache
    return c.data[c.page_table[b, t // 64], t % 64]


class _cus:
    """Temporarily plan for a different compute-unit count (changes the split)."""

    def __init__(self, n):
        self.n = n

    def __enter__(self):
        self.old = os.environ.get("MLA_NUM_CUS")
        os.environ["MLA_NUM_CUS"] = str(self.n)

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop("MLA_NUM_CUS", None)
        else:
            os.environ["MLA_NUM_CUS"] = self.old


SMALL = [
    # (seed, batch, heads, q_len, seq_lens)
    (101, 1, 16, 1, [256]),
    (102, 2, 16, 4, [300, 129]),
    (103, 3, 16, 2, [64, 65, 1000]),
    (104, 4, 32, 2, [17, 200, 640, 2051]),
    (105, 1, 8, 1, [1]),
    (106, 2, 4, 3, [3, 70]),
    (107, 5, 16, 4, [4, 5, 63, 64, 127]),
    (108, 2, 64, 1, [700, 90]),
    (109, 1, 1, 1, [333]),
    (110, 2, 32, 3, [500, 77]),      # 96 folded rows: eight waves
    (111, 1, 128, 1, [1000]),        # 128 folded rows
]


@pytest.mark.parametrize("seed,batch,heads,q_len,lens", SMALL, ids=[str(s[0]) for s in SMALL])
def test_decode_matches_oracle_small(seed, batch, heads, q_len, lens):
    case = synth.make_decode_case(seed, batch, heads, q_len, seq_lens=lens)
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, f"seed {seed}")


@pytest.mark.parametrize("cus", [1, 2, 3, 7, 64, 256, 1024])
def test_decode_split_plans_agree(cus):
    """Different compute-unit counts give different splits; all match the oracle."""
    case = synth.make_decode_case(201, 3, 16, 4, seq_lens=[1500, 64, 777])
    with _cus(cus):
        out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, f"cus {cus}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
@pytest.mark.parametrize("cus", [1, 2])
def test_decode_multi_window_shares(cus, kv_dtype):
    """148 pages on one or two workgroups: shares longer than the 128-page window of
    the tile list, request switches inside a window, and (one workgroup) the final
    output written by phase one itself."""
    case = synth.make_decode_case(208, 4, 16, 4, seq_lens=[5000, 64, 4000, 300], kv_dtype=kv_dtype)
    with _cus(cus):
        out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, f"cus {cus} {kv_dtype}")


def test_decode_workload0_full():
    case = synth.make_workload(0)
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, case.name)


def test_decode_ragged_many_requests():
    g = np.random.default_rng(5)
    lens = g.integers(2, 3000, size=37)
    case = synth.make_decode_case(202, 37, 16, 2, seq_lens=lens, max_seq_len=4096)
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, "ragged 37")


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_decode_more_requests_than_the_length_cache(kv_dtype):
    """600 requests: past the 512 lengths (and query offsets) the kernels cache in LDS, the
    shares read the rest from memory; many requests per share, short and ragged lengths."""
    g = np.random.default_rng(7)
    lens = g.integers(1, 400, size=600)
    case = synth.make_decode_case(211, 600, 16, 1, seq_lens=lens, max_seq_len=512, kv_dtype=kv_dtype)
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case, nthreads=min(16, os.cpu_count() or 1))
    assert_close(out, lse, ref_out, ref_lse, f"600 requests {kv_dtype}")


@pytest.mark.parametrize("cus", [1, 5, 256])
def test_decode_needle_bit_exact(cus):
    """q = 64 e_j and one row with value 32 at dim j: the needle's score leads every
    other by > 100 (natural units), all other weights underflow to 0 in fp32 and the
    output must be the needle's value columns bit for bit."""
    L = 3 * 64 + 17
    positions = [0, 63, 64, 127, 128, L - 1]
    batch = len(positions)
    case = synth.make_decode_case(301, batch, 16, 1, seq_lens=[L] * batch)
    g = np.random.default_rng(7)
    js = g.integers(0, 512, size=(batch, 16))
    for b, pos in enumerate(positions):
        for h in range(16):
            q = np.zeros(576, np.uint16)
            q[js[b, h]] = synth.bf16_bits(np.array([64.0], np.float32))[0]
            case.q[b, h] = q
        row = _row_bits(case, b, pos).copy()
        for h in range(16):
            row[js[b, h]] = synth.bf16_bits(np.array([32.0], np.float32))[0]
        _put_row(case, b, pos, row)
    with _cus(cus):
        out, lse = run_decode(case)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b, pos in enumerate(positions):
        want = _row_bits(case, b, pos)[:512]
        for h in range(16):
            assert np.array_equal(got[b, h], want), f"needle at {pos}, head {h}"


def test_decode_causal_needle():
    """A needle at row L-q+k is seen bit-exactly by drafts i >= k; drafts i < k match the oracle."""
    q_len, L, k = 4, 300, 2
    case = synth.make_decode_case(302, 1, 16, q_len, seq_lens=[L])
    pos = L - q_len + k
    j = 5
    for i in range(q_len):
        for h in range(16):
            qq = np.zeros(576, np.uint16)
            qq[j] = synth.bf16_bits(np.array([64.0], np.float32))[0]
            case.q[i, h] = qq
    row = _row_bits(case, 0, pos).copy()
    row[j] = synth.bf16_bits(np.array([32.0], np.float32))[0]
    _put_row(case, 0, pos, row)
    out, lse = run_decode(case)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for i in range(k, q_len):
        for h in range(16):
            assert np.array_equal(bits[i, h], _row_bits(case, 0, pos)[:512])
    ref_out, ref_lse = oracle.decode(case, tokens=list(range(k)))
    o, l_ = host(out, lse)
    assert_close(o[:k], l_[:k], ref_out, ref_lse, "drafts before the needle")


def test_decode_single_row_is_that_row():
    case = synth.make_decode_case(303, 3, 16, 1, seq_lens=[1, 1, 1])
    out, lse = run_decode(case)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(3):
        for h in range(16):
            assert np.array_equal(bits[b, h], _row_bits(case, b, 0)[:512])
    ref_out, ref_lse = oracle.decode(case)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-3


def test_decode_page_permutation_bitwise_invariant():
    a = synth.make_decode_case(304, 2, 16, 2, seq_lens=[900, 333])
    b = synth.make_decode_case(304, 2, 16, 2, seq_lens=[900, 333])
    # same logical rows, new physical placement
    c = b.cache
    perm = np.random.default_rng(11).permutation(c.num_pages)
    new_data = np.empty_like(c.data)
    new_data[perm] = c.data
    c.data = new_data
    c.page_table = perm[c.page_table].astype(np.int32)
    c.poison_page = int(perm[c.poison_page])
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)


def test_decode_deterministic():
    case = synth.make_decode_case(305, 4, 16, 4, seq_lens=[5000, 4000, 100, 2500])
    d = decode_inputs(case)
    o1, l1 = run_decode(case, d)
    o2, l2 = run_decode(case, d)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_nan_poison_has_no_effect():
    """Tails past each length and unused page-table entries point at NaN rows: the output
    must equal the run with finite poison bit for bit."""
    lens = [70, 129, 1]
    a = synth.make_decode_case(306, 3, 16, 1, seq_lens=lens, max_seq_len=400)
    b = synth.make_decode_case(306, 3, 16, 1, seq_lens=lens, max_seq_len=400, poison=synth.POISON_NAN)
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)
    assert torch.isfinite(ob.float()).all()


# The bf16 decode requests its first tile and query block before the lengths arrive,
# guessing that every request holds max_seq_len rows.  (seed, seq_lens, max_seq_len,
# cus): the guess right for every workgroup; wrong for every one (each request shorter,
# so most guessed pages lie past the lengths); right for the full-length requests only;
# more workgroups than pages (guessed tiles issued by workgroups whose share is empty).
GUESS_CASES = [(321, [2048] * 4, 2048, 64), (322, [700] * 4, 2048, 64),
               (323, [2048, 300, 2048, 1100], 2048, 48), (324, [64, 64], 2048, 256)]


@pytest.mark.parametrize("seed,lens,max_len,cus", GUESS_CASES, ids=["right", "wrong", "mixed", "idle"])
def test_decode_guessed_start(seed, lens, max_len, cus):
    """Parity with the oracle, and NaN rows in every page past the lengths (where the
    unused page-table entries point) leave the output bitwise unchanged."""
    a = synth.make_decode_case(seed, len(lens), 16, 4, seq_lens=lens, max_seq_len=max_len)
    b = synth.make_decode_case(seed, len(lens), 16, 4, seq_lens=lens, max_seq_len=max_len,
                               poison=synth.POISON_NAN)
    with _cus(cus):
        oa, la = run_decode(a)
        ob, lb = run_decode(b)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode(a)
    assert_close(*host(oa, la), ref_out, ref_lse, f"seed {seed}")
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)


# (seed, seq_lens, cus): plans that take each merge kernel.  Workgroups per request
# on average: 64 / 2 = 32 and 48 / 12 = 4 (the row-block merge, at most 40), 256 / 3
# (the per-row merge); 12 requests of 1-2 pages on 48 workgroups leave shares empty.
POISON_PLANS = [(311, [5000, 4000], 64), (312, [64, 65, 1, 128, 100, 3, 70, 127, 64, 2, 90, 33], 48),
                (313, [3000, 2500, 700], 256)]


@pytest.mark.parametrize("seed,lens,cus", POISON_PLANS, ids=["rows", "rows-sparse", "per-row"])
def test_decode_merge_reads_only_written_partials(seed, lens, cus):
    """The workspace starts as NaN bytes: both merge kernels read only the partials
    phase one wrote (empty shares take weight 0 and a written slot), so the output
    matches the oracle and is finite."""
    case = synth.make_decode_case(seed, len(lens), 16, 1, seq_lens=lens)
    d = decode_inputs(case)
    nb = mla.mla_splitkv_workspace_size(case.batch, case.heads, case.q_len, case.total_q(), case.max_seq_len,
                                        d["kind"])
    ws = torch.full((max(nb, 1),), 255, dtype=torch.uint8, device="cuda")
    with _cus(cus):
        out, lse = run_decode(case, d, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    ref_out, ref_lse = oracle.decode(case)
    assert_close(*host(out, lse), ref_out, ref_lse, f"seed {seed} cus {cus}")


def test_decode_short_workspace_is_rejected():
    case = synth.make_decode_case(307, 4, 16, 4, seq_lens=[4096] * 4)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        run_decode(case, workspace=ws)
    assert e.value.status == mla.MLA_ERR_WORKSPACE


def test_decode_workload1_sampled():
    """Full-size 64K-row decode (4 requests x 4 drafts x 16 heads), as benchmarked;
    the oracle evaluates one draft of each request, all heads."""
    case = synth.make_workload(1)
    out, lse = host(*run_decode(case))
    toks = [0, 5, 10, 15]  # request b, draft b
    ref_out, ref_lse = oracle.decode(case, tokens=toks, nthreads=min(16, os.cpu_count() or 1))
    errs = assert_close(out[toks], lse[toks], ref_out, ref_lse, case.name)
    print("workload1 sampled: max abs err %.3g, lse err %.3g, rel frob %.3g" % errs)


# ---------------------------------------------------------------- INT8 cache

INT8_SMALL = [
    # (seed, batch, heads, q_len, seq_lens)
    (501, 1, 16, 1, [256]),
    (502, 3, 16, 4, [65, 300, 1000]),
    (503, 4, 32, 2, [33, 64, 127, 2500]),
    (504, 2, 128, 1, [700, 90]),        # 128 folded rows: two row blocks
    (505, 1, 16, 4, [4]),
]


@pytest.mark.parametrize("seed,batch,heads,q_len,lens", INT8_SMALL, ids=[str(s[0]) for s in INT8_SMALL])
def test_decode_int8_matches_oracle(seed, batch, heads, q_len, lens):
    case = synth.make_decode_case(seed, batch, heads, q_len, seq_lens=lens, kv_dtype="int8")
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, f"int8 seed {seed}")


@pytest.mark.parametrize("cus", [1, 7, 256])
def test_decode_int8_split_plans_agree(cus):
    case = synth.make_decode_case(506, 3, 16, 2, seq_lens=[1500, 64, 777], kv_dtype="int8")
    with _cus(cus):
        out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, f"int8 cus {cus}")


def test_decode_int8_nan_scale_poison_has_no_effect():
    """Tail rows carry code 127 and a NaN scale: the output must not change."""
    lens = [70, 129, 1]
    a = synth.make_decode_case(507, 3, 16, 1, seq_lens=lens, max_seq_len=400, kv_dtype="int8")
    b = synth.make_decode_case(507, 3, 16, 1, seq_lens=lens, max_seq_len=400, kv_dtype="int8",
                               poison=synth.POISON_NAN)
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)
    assert torch.isfinite(ob.float()).all()


def test_decode_int8_page_permutation_bitwise_invariant():
    a = synth.make_decode_case(508, 2, 16, 2, seq_lens=[900, 333], kv_dtype="int8")
    b = synth.make_decode_case(508, 2, 16, 2, seq_lens=[900, 333], kv_dtype="int8")
    c = b.cache
    perm = np.random.default_rng(12).permutation(c.num_pages)
    nd, ns = np.empty_like(c.data), np.empty_like(c.scale)
    nd[perm] = c.data
    ns[perm] = c.scale
    c.data, c.scale = nd, ns
    c.page_table = perm[c.page_table].astype(np.int32)
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)


def test_decode_int8_needle():
    """A row whose score leads by > 100: the output is that row's dequantised values
    (the scale enters the value product through the bf16 probability, so the check is
    the tolerance, not bit equality)."""
    L = 200
    case = synth.make_decode_case(509, 2, 16, 1, seq_lens=[L, L], kv_dtype="int8")
    c = case.cache
    j = 7
    for b, pos in enumerate([5, L - 1]):
        for h in range(16):
            qq = np.zeros(576, np.uint16)
            qq[j] = synth.bf16_bits(np.array([64.0], np.float32))[0]
            case.q[b, h] = qq
        page, slot = c.page_table[b, pos // 64], pos % 64
        c.data[page, slot, j] = 127
        c.scale[page, slot] = np.float32(1.0)
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, "int8 needle")


@pytest.mark.parametrize("kv_dtype", ["int8", "fp8"])
@pytest.mark.parametrize("cus", [1, 2])
def test_decode_codes_window_restart(cus, kv_dtype):
    """INT8 / FP8 decode walks a share in windows of 256 staged page ids: 455 pages on
    one or two workgroups cross a window edge inside a request (20,000 rows), switch
    requests inside a window, and (one workgroup) write the final output directly."""
    case = synth.make_decode_case(510, 3, 16, 4, seq_lens=[20000, 64, 9000], kv_dtype=kv_dtype)
    with _cus(cus):
        out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, f"{kv_dtype} cus {cus} window restart")


# ---------------------------------------------------------------- FP8 (E4M3) cache

FP8_SMALL = [
    (521, 1, 16, 1, [256]),
    (522, 3, 16, 4, [65, 300, 1000]),
    (523, 4, 32, 2, [33, 64, 127, 2500]),
    (524, 2, 128, 1, [700, 90]),
    (525, 1, 16, 4, [4]),
]


@pytest.mark.parametrize("seed,batch,heads,q_len,lens", FP8_SMALL, ids=[str(s[0]) for s in FP8_SMALL])
def test_decode_fp8_matches_oracle(seed, batch, heads, q_len, lens):
    case = synth.make_decode_case(seed, batch, heads, q_len, seq_lens=lens, kv_dtype="fp8")
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, f"fp8 seed {seed}")


def test_decode_fp8_every_code():
    """Rows that hold every finite E4M3 code (subnormals, both zeros, +-448): the widening
    to bf16 must be exact for each of them."""
    case = synth.make_decode_case(526, 1, 16, 1, seq_lens=[300], kv_dtype="fp8")
    c = case.cache
    finite = np.array([v for v in range(256) if (v & 0x7F) != 0x7F], np.uint8)
    for t in range(300):
        c.data[c.page_table[0, t // 64], t % 64] = np.roll(np.resize(finite, 576), 7 * t)
    out, lse = host(*run_decode(case))
    ref_out, ref_lse = oracle.decode(case)
    assert_close(out, lse, ref_out, ref_lse, "fp8 every code")


def test_decode_fp8_nan_scale_poison_has_no_effect():
    lens = [70, 129, 1]
    a = synth.make_decode_case(527, 3, 16, 1, seq_lens=lens, max_seq_len=400, kv_dtype="fp8")
    b = synth.make_decode_case(527, 3, 16, 1, seq_lens=lens, max_seq_len=400, kv_dtype="fp8",
                               poison=synth.POISON_NAN)
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)
    assert torch.isfinite(ob.float()).all()


def test_decode_fp8_long_sampled():
    """Two 64K-row FP8 requests, 4 drafts x 16 heads; the oracle evaluates two tokens."""
    case = synth.make_decode_case(528, 2, 16, 4, seq_lens=[65536, 65536], kv_dtype="fp8")
    out, lse = host(*run_decode(case))
    toks = [0, 7]
    ref_out, ref_lse = oracle.decode(case, tokens=toks, nthreads=min(16, os.cpu_count() or 1))
    assert_close(out[toks], lse[toks], ref_out, ref_lse, "fp8 64K")


def test_decode_workload4_sampled():
    """Full-size INT8 decode (8 requests x 4 drafts x 16 heads, 262,144 rows each); the
    oracle evaluates one draft of two requests, all heads."""
    case = synth.make_workload(4)
    out, lse = host(*run_decode(case))
    toks = [0, 31]
    ref_out, ref_lse = oracle.decode(case, tokens=toks, nthreads=min(16, os.cpu_count() or 1))
    errs = assert_close(out[toks], lse[toks], ref_out, ref_lse, case.name)
    print("workload4 sampled: max abs err %.3g, lse err %.3g, rel frob %.3g" % errs)


def test_decode_workload2_sampled():
    """Ragged 16-request decode (lengths 32K-128K, 32 heads, 2 drafts); sampled rows."""
    case = synth.make_workload(2)
    out, lse = host(*run_decode(case))
    toks = [0, 13, 31]
    ref_out, ref_lse = oracle.decode(case, tokens=toks, nthreads=min(16, os.cpu_count() or 1))
    errs = assert_close(out[toks], lse[toks], ref_out, ref_lse, case.name)
    print("workload2 sampled: max abs err %.3g, lse err %.3g, rel frob %.3g" % errs)


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_decode_million_rows_sampled(kv_dtype):
    """Contexts of 1,048,576 and 700,001 rows (2 drafts, 16 heads): about 100-150 shares per
    request, so the merge reads its partials in several batches; the last draft of each
    request is checked against the oracle."""
    case = synth.make_decode_case(531, 2, 16, 2, seq_lens=[1 << 20, 700001], kv_dtype=kv_dtype)
    out, lse = host(*run_decode(case))
    toks = [1, 3]
    ref_out, ref_lse = oracle.decode(case, tokens=toks, nthreads=min(16, os.cpu_count() or 1))
    errs = assert_close(out[toks], lse[toks], ref_out, ref_lse, f"1M rows {kv_dtype}")
    print("million rows %s: max abs err %.3g, lse err %.3g, rel frob %.3g" % ((kv_dtype,) + errs))


def test_decode_fp8_nan_code_tail_has_no_effect():
    """Rows past each request's end (and the poison page) hold the E4M3 NaN code 0x7F with a
    NaN scale: the output must equal the run with finite poison bit for bit."""
    lens = [70, 129, 1, 4000]
    a = synth.make_decode_case(529, 4, 16, 1, seq_lens=lens, max_seq_len=4096, kv_dtype="fp8")
    b = synth.make_decode_case(529, 4, 16, 1, seq_lens=lens, max_seq_len=4096, kv_dtype="fp8")
    c = b.cache
    for bb, L in enumerate(lens):
        n = (L + 63) // 64
        c.data[c.page_table[bb, n - 1], L - 64 * (n - 1):] = 0x7F
        c.scale[c.page_table[bb, n - 1], L - 64 * (n - 1):] = np.float32("nan")
    c.data[c.poison_page] = 0x7F
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)
    assert torch.isfinite(ob.float()).all()
