"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes the oracle to an independent fact: the unabsorbed MLA form
computed separately in numpy, brute-force softmax in pure Python, closed-form
cases, invariants (split/merge, page permutation, causal truncation) and
special cases.  ``test_oracle_mutants`` plants plausible mistakes in a copy of
the oracle's C source and checks that these pins catch every one.
"""
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")
SCALE = 1.0 / math.sqrt(192.0)


def _bf16(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


def _f(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------
# helpers that build small oracle calls directly
# --------------------------------------------------------------------------

def _contiguous_call(q_bits, rows_bits, n_new, page_size=4, perm=None, lib=None, bounds=None,
                     kv_scale=None, dv=None):
    """One request whose cache rows are ``rows_bits`` [L, dqk], paged with ``perm``."""
    L, dqk = rows_bits.shape
    npages = (L + page_size - 1) // page_size
    pool = npages + 1
    if perm is None:
        perm = np.arange(pool)
    dt = rows_bits.dtype
    pages = np.zeros((pool, page_size, dqk), dtype=dt)
    sc = None if kv_scale is None else np.zeros((pool, page_size), dtype=np.float32)
    pt = np.zeros((1, npages), dtype=np.int32)
    for j in range(npages):
        phys = int(perm[j])
        pt[0, j] = phys
        chunk = rows_bits[j * page_size:(j + 1) * page_size]
        pages[phys, :chunk.shape[0]] = chunk
        if sc is not None:
            sc[phys, :chunk.shape[0]] = kv_scale[j * page_size:(j + 1) * page_size]
    q_start = np.array([0, n_new], dtype=np.int32)
    kv_len = np.array([L], dtype=np.int32)
    return oracle.attention(q_bits, pages, sc, pt, q_start, kv_len, SCALE,
                            dv=dv if dv is not None else min(512, dqk), bounds=bounds, lib=lib)


def _rand_case(seed, L, n_new, H, dqk=576, scale_rows=1.0):
    g = np.random.default_rng(seed)
    q = _bf16(g.standard_normal((n_new, H, dqk)))
    rows = _bf16(g.standard_normal((L, dqk)) * scale_rows)
    return q, rows


# --------------------------------------------------------------------------
# 1. Absorbed == unabsorbed MLA (the published formulation, computed in numpy)
# --------------------------------------------------------------------------

def _unabsorbed_check(seed, H, L, n_new, d_lat, d_rope, d_head, lib=None):
    """Unabsorbed: per head k = [W_UK c; k_rope], q = [q_nope; q_rope], v = W_UV c,
    ordinary softmax attention with scale 1/sqrt(d_head + d_rope).  Absorbed:
    q_abs = [W_UK^T q_nope; q_rope] against the latent row [c; k_rope]; the oracle's
    latent output, up-projected by W_UV, must equal the unabsorbed head output."""
    g = np.random.default_rng(seed)
    # Small integers keep the absorbed query exactly representable in bf16.
    W_UK = g.integers(-1, 2, size=(H, d_head, d_lat)).astype(np.float64)
    W_UV = g.standard_normal((H, d_head, d_lat))
    q_nope = g.integers(-1, 2, size=(n_new, H, d_head)).astype(np.float64)
    q_rope = _f(_bf16(g.standard_normal((n_new, H, d_rope))))
    c = _f(_bf16(g.standard_normal((L, d_lat)) * 0.125))
    k_rope = _f(_bf16(g.standard_normal((L, d_rope))))
    scale = 1.0 / math.sqrt(d_head + d_rope)

    # unabsorbed multi-head attention, causal over the new tokens
    o_ref = np.zeros((n_new, H, d_head))
    lse_ref = np.zeros((n_new, H))
    for i in range(n_new):
        vis = L - n_new + i + 1
        for h in range(H):
            k = np.concatenate([c[:vis] @ W_UK[h].T, k_rope[:vis]], axis=1)     # [vis, d_head+d_rope]
            qh = np.concatenate([q_nope[i, h], q_rope[i, h]])
            v = c[:vis] @ W_UV[h].T                                             # [vis, d_head]
            s = scale * (k @ qh)
            m = s.max()
            lse_ref[i, h] = m + math.log(np.exp(s - m).sum())
            o_ref[i, h] = (np.exp(s - lse_ref[i, h])[:, None] * v).sum(0)

    # absorbed inputs for the oracle
    q_abs = np.concatenate([np.einsum("hdl,ihd->ihl", W_UK, q_nope), q_rope], axis=2)
    assert np.abs(q_abs).max() <= 256  # integers below 256 and bf16 values: exact
    q_bits = _bf16(q_abs)
    assert np.array_equal(_f(q_bits), q_abs)
    rows_bits = _bf16(np.concatenate([c, k_rope], axis=1))
    pt = np.arange((L + 63) // 64, dtype=np.int32)[None]
    pages = np.zeros((pt.shape[1], 64, d_lat + d_rope), dtype=np.uint16)
    pages.reshape(-1, d_lat + d_rope)[:L] = rows_bits
    out, lse = oracle.attention(q_bits, pages, None, pt, np.array([0, n_new], np.int32),
                                np.array([L], np.int32), scale, dv=d_lat, lib=lib)
    o_abs = np.einsum("hdl,ihl->ihd", W_UV, out)
    return o_abs, o_ref, lse, lse_ref


def test_unabsorbed_identity_full_dims():
    o_abs, o_ref, lse, lse_ref = _unabsorbed_check(11, H=4, L=150, n_new=3, d_lat=512, d_rope=64,
                                                    d_head=128)
    np.testing.assert_allclose(o_abs, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_unabsorbed_identity_small_dims():
    o_abs, o_ref, lse, lse_ref = _unabsorbed_check(12, H=3, L=9, n_new=2, d_lat=16, d_rope=4,
                                                    d_head=8)
    np.testing.assert_allclose(o_abs, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# 2. Brute-force softmax in pure Python (no max shift, exact summation)
# --------------------------------------------------------------------------

def _brute(qf, rowsf, n_new, dv, scale):
    L = len(rowsf)
    outs, lses = [], []
    for i, qi in enumerate(qf):
        vis = L - n_new + i + 1
        o_h, l_h = [], []
        for qh in qi:
            e = [math.exp(scale * math.fsum(a * b for a, b in zip(qh, rowsf[t]))) for t in range(vis)]
            z = math.fsum(e)
            o_h.append([math.fsum(e[t] * rowsf[t][d] for t in range(vis)) / z for d in range(dv)])
            l_h.append(math.log(z))
        outs.append(o_h)
        lses.append(l_h)
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("L,n_new,H,dqk,dv,seed", [(1, 1, 1, 5, 3, 0), (7, 3, 2, 6, 4, 1),
                                                   (13, 2, 3, 9, 7, 2), (20, 5, 1, 12, 12, 3)])
def test_bruteforce_softmax(L, n_new, H, dqk, dv, seed):
    q, rows = _rand_case(seed, L, n_new, H, dqk)
    out, lse = _contiguous_call(q, rows, n_new, page_size=3, dv=dv)
    bo, bl = _brute(_f(q).tolist(), _f(rows).tolist(), n_new, dv, SCALE)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-13, atol=1e-13)


def test_probabilities_sum_to_one():
    """sum_t exp(s_t - lse) = 1, checked with the pure-Python scores and the oracle's lse."""
    q, rows = _rand_case(5, 40, 2, 2, 576)
    _, lse = _contiguous_call(q, rows, 2, page_size=8)
    qf, rf = _f(q), _f(rows)
    for i in range(2):
        vis = 40 - 2 + i + 1
        for h in range(2):
            s = [SCALE * math.fsum(qf[i, h] * rf[t]) for t in range(vis)]
            assert abs(math.fsum(math.exp(x - lse[i, h]) for x in s) - 1.0) < 1e-13


# --------------------------------------------------------------------------
# 3. Closed-form golden cases
# --------------------------------------------------------------------------

def _eval(expr):
    return float(eval(str(expr), {"__builtins__": {}}, {"e": math.e, "log": math.log,
                                                         "exp": math.exp}))


def _golden_cases():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_closed_form(case, lib=None):
    _run_golden(case, lib)


def _run_golden(case, lib=None):
    q = _bf16(np.array(case["q"], dtype=np.float32))
    if case["kv_dtype"] == "int8":
        pages = np.array(case["pages"], dtype=np.int8)
        scales = np.array(case["scales"], dtype=np.float32)
    else:
        pages = _bf16(np.array(case["pages"], dtype=np.float32))
        assert np.array_equal(_f(pages), np.array(case["pages"], dtype=np.float64))
        scales = None
    out, lse = oracle.attention(q, pages, scales, np.array(case["page_table"], np.int32),
                                np.array(case["q_start"], np.int32),
                                np.array(case["kv_len"], np.int32),
                                _eval(case["softmax_scale"]), dv=case["dv"], lib=lib)
    exp_out = np.vectorize(_eval, otypes=[float])(np.array(case["expect_out"], dtype=object))
    exp_lse = np.vectorize(_eval, otypes=[float])(np.array(case["expect_lse"], dtype=object))
    np.testing.assert_allclose(out, exp_out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, exp_lse, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# 4. Invariants: split/merge, page permutation, causal truncation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bounds", [[0, 100], [0, 1, 100], [0, 30, 30, 64, 99, 100],
                                    [0, 5, 17, 18, 40, 41, 50, 100], [0, 64, 65, 66, 100]])
def test_split_merge_equals_unsplit(bounds):
    """Partials over any partition, merged by their lse, equal the unsplit result.
    With 4 drafts on 66 rows, the ranges past a draft's causal limit are empty for it."""
    case = synth.make_decode_case(21, batch=2, heads=3, q_len=4, seq_lens=[66, 31])
    o1, l1 = oracle.decode(case)
    o2, l2 = oracle.decode(case, bounds=bounds)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-13)


def test_page_permutation_invariance_bit_identical():
    q, rows = _rand_case(31, 300, 3, 2, 576)
    o1, l1 = _contiguous_call(q, rows, 3, page_size=64)
    perm = np.random.default_rng(3).permutation(6)
    o2, l2 = _contiguous_call(q, rows, 3, page_size=64, perm=perm)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # and against a single flat page
    o3, l3 = _contiguous_call(q, rows, 3, page_size=300)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_causal_rows_equal_truncated_single_token_calls():
    """Draft i of a q_len=4 call equals a q_len=1 call on the first L-3+i rows."""
    q, rows = _rand_case(41, 90, 4, 3, 576)
    out, lse = _contiguous_call(q, rows, 4, page_size=64)
    for i in range(4):
        oi, li = _contiguous_call(q[i:i + 1], rows[:90 - 3 + i], 1, page_size=64)
        assert np.array_equal(out[i], oi[0]) and np.array_equal(lse[i], li[0])


def test_prefill_rows_equal_decode_rows():
    """Token j of prefill request b equals decode with q_len=1 on its first P_b+j+1 rows."""
    case = synth.make_prefill_case(51, heads=2, prefix_lens=[70, 0, 5], new_lens=[6, 9, 1])
    out, lse = oracle.prefill(case)
    c = case.cache
    for b in range(case.batch):
        for j in range(int(case.cu_seqlens_q[b + 1] - case.cu_seqlens_q[b])):
            tok = int(case.cu_seqlens_q[b]) + j
            L = int(case.prefix_lens[b]) + j + 1
            od, ld = oracle.attention(case.q[tok:tok + 1], c.data, None, c.page_table[b:b + 1],
                                      np.array([0, 1], np.int32), np.array([L], np.int32), SCALE)
            assert np.array_equal(out[tok], od[0]) and np.array_equal(lse[tok], ld[0])


# --------------------------------------------------------------------------
# 5. Special cases
# --------------------------------------------------------------------------

def test_single_row_returns_that_row():
    q, rows = _rand_case(61, 1, 1, 4, 576)
    out, lse = _contiguous_call(q, rows, 1)
    rf, qf = _f(rows), _f(q)
    for h in range(4):
        assert np.array_equal(out[0, h], rf[0, :512])
        assert abs(lse[0, h] - SCALE * math.fsum(qf[0, h] * rf[0])) < 1e-12


def test_zero_query_gives_mean_of_values():
    L = 37
    _, rows = _rand_case(62, L, 1, 1, 576)
    q = np.zeros((1, 2, 576), dtype=np.uint16)
    out, lse = _contiguous_call(q, rows, 1, page_size=8)
    np.testing.assert_allclose(out[0, 0], _f(rows)[:, :512].mean(0), rtol=1e-12, atol=1e-14)
    assert abs(lse[0, 0] - math.log(L)) < 1e-13


def test_equal_rows_give_that_row():
    _, rows = _rand_case(63, 1, 1, 1, 576)
    rows = np.repeat(rows, 25, axis=0)
    q, _ = _rand_case(64, 1, 1, 3, 576)
    out, lse = _contiguous_call(q, rows, 1, page_size=4)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], _f(rows)[0, :512], rtol=1e-13, atol=1e-14)


def test_int8_unit_scale_equals_bf16_on_integers():
    g = np.random.default_rng(71)
    codes = g.integers(-127, 128, size=(50, 576)).astype(np.int8)
    q = _bf16(g.standard_normal((2, 2, 576)) * 0.01)
    o8, l8 = _contiguous_call(q, codes, 2, page_size=16, kv_scale=np.ones(50, np.float32))
    ob, lb = _contiguous_call(q, _bf16(codes.astype(np.float32)), 2, page_size=16)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_int8_scale_is_per_row():
    """Scaling row t's codes by 2 and its scale by 1/2 changes nothing (exact in fp64)."""
    g = np.random.default_rng(72)
    codes = g.integers(-60, 61, size=(20, 576)).astype(np.int8)
    sc = (g.random(20) + 0.5).astype(np.float32) * np.float32(0.01)
    q = _bf16(g.standard_normal((1, 2, 576)))
    o1, l1 = _contiguous_call(q, codes, 1, page_size=8, kv_scale=sc)
    codes2 = codes.copy()
    codes2[3] = codes[3] * 2
    sc2 = sc.copy()
    sc2[3] = sc[3] / np.float32(2)
    o2, l2 = _contiguous_call(q, codes2, 1, page_size=8, kv_scale=sc2)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-15)


def test_oracle_rejects_out_of_range_page():
    q, rows = _rand_case(81, 10, 1, 1, 576)
    pages = np.zeros((1, 64, 576), np.uint16)
    with pytest.raises(ValueError):
        oracle.attention(q, pages, None, np.array([[5]], np.int32), np.array([0, 1], np.int32),
                         np.array([10], np.int32), SCALE)


# --------------------------------------------------------------------------
# 6. Planted mistakes: every mutant of the oracle must fail some pin
# --------------------------------------------------------------------------

MUTANTS = [
    ("off_by_one_causal", "int last = L - n_b + i;", "int last = L - n_b + i - 1;"),
    ("causal_top_left", "int last = L - n_b + i;", "int last = i < L ? i : L - 1;"),
    ("dropped_rope_columns", "for (int d = 0; d < j->dqk; ++d) acc += qd[d] * c[d];",
     "for (int d = 0; d < j->dv; ++d) acc += qd[d] * c[d];"),
    ("swapped_page_index", "int pj = t / j->page_size, slot = t % j->page_size;",
     "int slot = t / j->page_size, pj = t % j->page_size;"),
    ("lse_log2", "double lse = m + log(sum);", "double lse = m + log2(sum);"),
    ("scale_dropped", "s[t - lo] = j->softmax_scale * acc;", "s[t - lo] = acc;"),
    ("int8_scale_dropped", "c[d] = (double)row[d] * s;", "c[d] = (double)row[d];"),
    ("merge_unnormalised", "double w = exp(part_lse[k] - total);", "double w = exp(part_lse[k] - m);"),
    ("value_from_rope_end", "for (int d = 0; d < j->dv; ++d) o[d] += w * c[d];",
     "for (int d = 0; d < j->dv; ++d) o[d] += w * c[d + (j->dqk - j->dv)];"),
    ("query_head_stride", "const uint16_t *qr = j->q + ((size_t)tok * j->H + h) * j->dqk;",
     "const uint16_t *qr = j->q + ((size_t)h * j->H + tok % j->H) * j->dqk;"),
]


def _pins_pass(lib):
    """Run a battery of pins against a given oracle library; True when all pass."""
    try:
        for case in _golden_cases():
            _run_golden(case, lib)
        o_abs, o_ref, lse, lse_ref = _unabsorbed_check(12, H=3, L=9, n_new=2, d_lat=16, d_rope=4,
                                                        d_head=8, lib=lib)
        np.testing.assert_allclose(o_abs, o_ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
        q, rows = _rand_case(1, 7, 3, 2, 6)
        out, l_ = _contiguous_call(q, rows, 3, page_size=3, dv=4, lib=lib)
        bo, bl = _brute(_f(q).tolist(), _f(rows).tolist(), 3, 4, SCALE)
        np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l_, bl, rtol=1e-13, atol=1e-13)
        case = synth.make_decode_case(21, batch=2, heads=3, q_len=4, seq_lens=[66, 31])
        c = case.cache
        args = (case.q, c.data, c.scale, c.page_table, case.q_start(), c.kv_lens, SCALE)
        o1, l1 = oracle.attention(*args, lib=lib)
        o2, l2 = oracle.attention(*args, bounds=[0, 5, 17, 64, 100], lib=lib)
        np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-13)
    except (AssertionError, ValueError):
        return False
    return True


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_oracle_mutants_are_caught(name, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"libmut_{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", str(path),
                           "-o", str(so), "-lm"])
    lib = oracle.load_library(str(so))
    assert not _pins_pass(lib), f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_battery():
    assert _pins_pass(oracle._load())
