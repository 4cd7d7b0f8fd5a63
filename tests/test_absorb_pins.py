"""Pins of the absorption / up-projection oracle (CPU): facts the definitions fix,
checked without retyping them, plus planted mistakes that must fail.

[MLA] (DeepSeek-V2): per head, k_nope = W_UK[h] c and v = W_UV[h] c for a latent row
c; absorbed, the query is [W_UK[h]^T q_nope; q_rope] and the head output is W_UV[h]
applied to the latent attention output."""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle.absorb import D_LAT, D_NOPE, D_ROPE, D_V, mha_unabsorbed, q_absorb, v_up


def _bits(x):
    return synth.bf16_bits(np.asarray(x, np.float32))


def _vals(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def _check_absorb(fn):
    rng = np.random.default_rng(1)
    T, H = 3, 2
    q = _bits(rng.standard_normal((T, H, D_NOPE + D_ROPE)))
    # identity weights: W_UK[h][d][c] = [c == d] -> q_abs = [q_nope, 0 ...] and the rope passes
    w = np.zeros((H, D_NOPE, D_LAT), np.float32)
    w[:, np.arange(D_NOPE), np.arange(D_NOPE)] = 1.0
    out = fn(q, _bits(w))
    assert out.shape == (T, H, D_LAT + D_ROPE)
    assert np.array_equal(out[..., :D_NOPE], _vals(q)[..., :D_NOPE])
    assert np.all(out[..., D_NOPE:D_LAT] == 0)
    assert np.array_equal(out[..., D_LAT:], _vals(q)[..., D_NOPE:])
    # a different permutation per head: W_UK[h][d][pi_h(d)] = 1 moves q_nope[d] to column pi_h(d)
    w = np.zeros((H, D_NOPE, D_LAT), np.float32)
    perms = [rng.permutation(D_LAT)[:D_NOPE] for _ in range(H)]
    for h in range(H):
        w[h, np.arange(D_NOPE), perms[h]] = 1.0
    out = fn(q, _bits(w))
    for h in range(H):
        assert np.array_equal(out[:, h, perms[h]], _vals(q)[:, h, :D_NOPE])
    # brute force: the score identity q_abs . c == q_nope . (W_UK c) for one (t, h)
    w = _bits(rng.standard_normal((H, D_NOPE, D_LAT)) * 0.1)
    c = rng.standard_normal(D_LAT)
    out = fn(q, w)
    wv, qv = _vals(w), _vals(q)
    t, h = 2, 1
    k_nope = [sum(wv[h, d, j] * c[j] for j in range(D_LAT)) for d in range(D_NOPE)]
    lhs = sum(qv[t, h, d] * k_nope[d] for d in range(D_NOPE))
    rhs = sum(out[t, h, j] * c[j] for j in range(D_LAT))
    assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))


def _check_up(fn):
    rng = np.random.default_rng(2)
    T, H = 3, 2
    o = rng.standard_normal((T, H, D_LAT))
    w = np.zeros((H, D_V, D_LAT), np.float32)
    w[:, np.arange(D_V), np.arange(D_V) + 7] = 1.0                 # W_UV picks latent columns 7 .. 134
    out = fn(o, _bits(w))
    assert out.shape == (T, H, D_V)
    assert np.array_equal(out, o[..., 7:7 + D_V])
    w = _bits(rng.standard_normal((H, D_V, D_LAT)))
    out = fn(o, w)
    wv = _vals(w)
    t, h, v = 1, 1, 5
    ref = sum(wv[h, v, j] * o[t, h, j] for j in range(D_LAT))
    assert abs(out[t, h, v] - ref) <= 1e-9 * (1 + abs(ref))
    # bf16 bits are widened exactly
    ob = _bits(o)
    assert np.array_equal(fn(ob, w), fn(_vals(ob), w))


def test_absorb_pins():
    _check_absorb(q_absorb)


def test_up_projection_pins():
    _check_up(v_up)


def _absorb_transposed(q_bits, w_bits):   # contracts the latent index instead of the nope index
    q = _vals(q_bits)
    w = _vals(w_bits)
    qa = np.einsum("hdc,thc->thd", w, np.pad(q[..., :D_NOPE], ((0, 0), (0, 0), (0, D_LAT - D_NOPE))))
    return np.concatenate([np.pad(qa, ((0, 0), (0, 0), (0, D_LAT - D_NOPE))), q[..., D_NOPE:]], axis=2)


def _absorb_no_rope(q_bits, w_bits):
    out = q_absorb(q_bits, w_bits)
    out[..., D_LAT:] = 0
    return out


def _absorb_head_swap(q_bits, w_bits):
    return q_absorb(q_bits, w_bits[::-1].copy())


@pytest.mark.parametrize("mutant", [_absorb_transposed, _absorb_no_rope, _absorb_head_swap])
def test_absorb_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        _check_absorb(mutant)


def _up_head_swap(o, w_bits):
    return v_up(o, w_bits[::-1].copy())


def _up_offset(o, w_bits):   # reads the latent columns shifted by one
    o = _vals(o) if np.asarray(o).dtype == np.uint16 else np.asarray(o, np.float64)
    return v_up(np.roll(o, 1, axis=2), w_bits)


@pytest.mark.parametrize("mutant", [_up_head_swap, _up_offset])
def test_up_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        _check_up(mutant)


# ---------------- the unabsorbed attention ----------------

def _case(seed, H, lens, n_new, int_weights):
    g = np.random.default_rng(seed)
    if int_weights:   # small integers: the absorbed query stays exact in bf16
        w_uk = _bits(g.integers(-1, 2, size=(H, D_NOPE, D_LAT)))
        q = _bits(np.concatenate([g.integers(-1, 2, size=(sum(n_new), H, D_NOPE)),
                                  g.standard_normal((sum(n_new), H, D_ROPE))], axis=2))
    else:
        w_uk = _bits(g.standard_normal((H, D_NOPE, D_LAT)) * 0.05)
        q = _bits(g.standard_normal((sum(n_new), H, D_NOPE + D_ROPE)))
    w_uv = _bits(g.standard_normal((H, D_V, D_LAT)) * 0.05)
    lat = [_bits(g.standard_normal((L, D_LAT)) * 0.125) for L in lens]
    rope = [_bits(g.standard_normal((L, D_ROPE))) for L in lens]
    q_start = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    return q, lat, rope, w_uk, w_uv, q_start, np.asarray(lens, np.int32)


def test_unabsorbed_single_row_and_equal_keys():
    """One visible row: the output is that row's value exactly.  Equal keys: the softmax is
    uniform, so the output is the mean of the values and lse = s + ln(count)."""
    q, lat, rope, w_uk, w_uv, qs, lens = _case(3, 2, [1], [1], False)
    out, lse = mha_unabsorbed(q, lat, rope, w_uk, w_uv, qs, lens, 0.1)
    v = np.einsum("hvc,c->hv", _vals(w_uv), _vals(lat[0])[0])
    np.testing.assert_allclose(out[0], v, rtol=1e-12, atol=1e-14)
    q, lat, rope, w_uk, w_uv, qs, lens = _case(4, 2, [5], [1], False)
    lat[0][:] = lat[0][0]
    rope[0][:] = rope[0][0]
    out, lse = mha_unabsorbed(q, lat, rope, w_uk, w_uv, qs, lens, 0.1)
    v = np.einsum("hvc,c->hv", _vals(w_uv), _vals(lat[0])[0])
    np.testing.assert_allclose(out[0], v, rtol=1e-12, atol=1e-14)
    k = np.concatenate([_vals(w_uk)[0] @ _vals(lat[0])[0], _vals(rope[0])[0]])
    assert abs(lse[0, 0] - (0.1 * (k @ _vals(q)[0, 0]) + math.log(5))) <= 1e-12


def test_unabsorbed_equals_absorbed_attention_oracle():
    """q_absorb -> the latent attention oracle -> v_up equals the unabsorbed definition
    (small integer W_UK and q_nope keep the absorbed query exact in bf16)."""
    H, lens, n_new = 3, [150, 70], [3, 2]
    q, lat, rope, w_uk, w_uv, qs, kv = _case(5, H, lens, n_new, True)
    scale = 1.0 / math.sqrt(D_NOPE + D_ROPE)
    ref, ref_lse = mha_unabsorbed(q, lat, rope, w_uk, w_uv, qs, kv, scale)
    q_abs = q_absorb(q, w_uk)
    q_bits = _bits(q_abs)
    assert np.array_equal(_vals(q_bits), q_abs)
    pages = []
    pt = np.zeros((len(lens), max((L + 63) // 64 for L in lens)), np.int32)
    n = 0
    for b, L in enumerate(lens):
        rows = np.concatenate([lat[b], rope[b]], axis=1)
        np_b = (L + 63) // 64
        blk = np.zeros((np_b * 64, D_LAT + D_ROPE), np.uint16)
        blk[:L] = rows
        pages.append(blk.reshape(np_b, 64, -1))
        pt[b, :np_b] = np.arange(n, n + np_b)
        n += np_b
    o_lat, lse = oracle.attention(q_bits, np.concatenate(pages), None, pt, qs, kv, scale)
    out = v_up(o_lat, w_uv)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
