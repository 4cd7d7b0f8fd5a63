"""Pins of the KV-append oracle (CPU): what the definition of the step fixes,
checked without retyping its formulas, plus planted mistakes that must fail.

The step writes new rows to logical positions of the paged cache and, for an
INT8 cache, encodes each row symmetrically with one fp32 scale ([TALK]
"构建面向 Agentic 推理的下一代 LLM 推理引擎", section "Kernel：让 MLA 真正跑满
GPU": paged latent cache, INT8 latent cache; the encoding value = code *
scale is the one the attention entry points read)."""
import numpy as np
import pytest

import oracle
import synth
from oracle.kv_append import bf16_bits_to_f32


def _bf16_row(rng, n=576, std=1.0):
    return synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(std)))


# ---------------- quantisation ----------------

def _check_quantizer(q):
    """Raise AssertionError when the quantiser breaks a property the definition fixes."""
    rng = np.random.default_rng(5)
    for std in (1.0, 1e-3, 37.0):
        for _ in range(20):
            x = _bf16_row(rng, std=std)
            codes, scale = q(x)
            codes = codes.astype(np.int32)
            scale = np.float32(scale)
            i = int(np.argmax(np.abs(x)))
            assert codes[i] == (127 if x[i] > 0 else -127)                    # the max maps to +-127
            assert np.all(np.abs(codes) <= 127)
            err = np.abs(codes.astype(np.float64) * np.float64(scale) - x.astype(np.float64))
            # nearest code of the fp32 quotient: |x / scale| <= 127, so the division
            # itself may move the quotient by up to 127 * 2^-24 before rounding
            assert np.all(err <= (0.5 + 127 * 2.0 ** -24) * np.float64(scale) * (1 + 1e-6))
            assert abs(np.float64(scale) * 127 - np.max(np.abs(x))) <= 2 ** -22 * np.max(np.abs(x))
            # homogeneity: a power-of-two factor moves the scale, not the codes
            c2, s2 = q(x * np.float32(8.0))
            assert np.array_equal(c2.astype(np.int32), codes) and np.float32(s2) == np.float32(8.0) * scale
            # sign symmetry
            c3, s3 = q(-x)
            assert np.array_equal(c3.astype(np.int32), -codes) and np.float32(s3) == scale
    # ties go to the even code: with max|x| = 127 the scale is exactly 1
    x = np.zeros(576, np.float32)
    x[:8] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 126.5, -1.5]
    codes, scale = q(x)
    assert np.float32(scale) == np.float32(1.0)
    assert codes[:8].astype(np.int32).tolist() == [127, 2, 4, -2, -4, 0, 126, -2]
    # an all-zero row: codes 0, scale 1 (reads back as zeros)
    codes, scale = q(np.zeros(576, np.float32))
    assert np.all(codes == 0) and np.float32(scale) == np.float32(1.0)


def test_quantizer_pins():
    _check_quantizer(oracle.quantize_row)


def _trunc(x):
    x = np.asarray(x, np.float32)
    s = np.float32(np.max(np.abs(x)) / np.float32(127.0)) or np.float32(1.0)
    return np.clip(np.trunc(x / s), -127, 127).astype(np.int8), s


def _div128(x):
    x = np.asarray(x, np.float32)
    s = np.float32(np.max(np.abs(x)) / np.float32(128.0)) or np.float32(1.0)
    return np.clip(np.rint(x / s), -127, 127).astype(np.int8), s


def _half_away(x):
    x = np.asarray(x, np.float32)
    s = np.float32(np.max(np.abs(x)) / np.float32(127.0)) or np.float32(1.0)
    y = x / s
    return np.clip(np.sign(y) * np.floor(np.abs(y) + 0.5), -127, 127).astype(np.int8), s


def _mean_scale(x):
    x = np.asarray(x, np.float32)
    s = np.float32(np.mean(np.abs(x)) * 3 / np.float32(127.0)) or np.float32(1.0)
    return np.clip(np.rint(x / s), -127, 127).astype(np.int8), s


def _zero_scale0(x):
    x = np.asarray(x, np.float32)
    s = np.float32(np.max(np.abs(x)) / np.float32(127.0))
    with np.errstate(invalid="ignore", divide="ignore"):
        c = np.nan_to_num(np.rint(x / s))
    return np.clip(c, -127, 127).astype(np.int8), s


@pytest.mark.parametrize("mutant", [_trunc, _div128, _half_away, _mean_scale, _zero_scale0],
                         ids=lambda f: f.__name__)
def test_quantizer_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        _check_quantizer(mutant)


# ---------------- placement ----------------

def _setup(rng, kv_dtype, batch=3, max_pages=6):
    num_pages = batch * max_pages + 2
    perm = rng.permutation(num_pages - 1)[: batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    if kv_dtype == "bf16":
        cache = rng.integers(0, 1 << 16, size=(num_pages, 64, 576), dtype=np.uint16)
        scale = None
    else:
        cache = rng.integers(-127, 128, size=(num_pages, 64, 576), dtype=np.int8)
        scale = rng.random((num_pages, 64), dtype=np.float32) + np.float32(0.5)
    start = np.array([0, 63, 130], np.int32)[:batch]
    n = np.array([5, 70, 3], np.int32)[:batch]
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    new = synth.bf16_bits(rng.standard_normal((int(cu[-1]), 576)).astype(np.float32))
    return cache, scale, perm, start, cu, new


def _logical(cache, perm, b, t):
    return cache[perm[b, t // 64], t % 64]


def _check_placement(append, kv_dtype):
    rng = np.random.default_rng(11)
    cache, scale, perm, start, cu, new = _setup(rng, kv_dtype)
    out, sc = append(new, cu, start, cache, scale, kv_dtype, perm)
    written = set()
    for b in range(len(start)):
        for j in range(int(cu[b + 1] - cu[b])):
            t = int(start[b]) + j
            written.add((int(perm[b, t // 64]), t % 64))
            row = new[cu[b] + j]
            if kv_dtype == "bf16":
                assert np.array_equal(_logical(out, perm, b, t), row)
            else:  # reads back within half a code step of the bf16 value
                x = bf16_bits_to_f32(row).astype(np.float64)
                val = _logical(out, perm, b, t).astype(np.float64) * np.float64(sc[perm[b, t // 64], t % 64])
                assert np.max(np.abs(val - x)) <= (0.5 + 127 * 2.0 ** -24) * np.max(np.abs(x)) / 127 * (1 + 1e-5)
    for p in range(cache.shape[0]):
        for s in range(64):
            if (p, s) not in written:
                assert np.array_equal(out[p, s], cache[p, s])
                if sc is not None:
                    assert sc[p, s] == scale[p, s]
    # rows past the page table are dropped and nothing else changes
    far = np.array([perm.shape[1] * 64 - 2, 0, 0], np.int32)
    cu2 = np.array([0, 5, 5, 5], np.int32)
    out2, _ = append(new[:5], cu2, far, cache, scale, kv_dtype, perm)
    changed = {(p, s) for p in range(cache.shape[0]) for s in range(64) if not np.array_equal(out2[p, s], cache[p, s])}
    t0 = int(far[0])
    assert changed <= {(int(perm[0, (t0 + k) // 64]), (t0 + k) % 64) for k in range(2)}


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_placement_pins(kv_dtype):
    _check_placement(oracle.kv_append, kv_dtype)


def _swapped(new, cu, start, cache, scale, kv_dtype, pt):
    # page and slot taken from the wrong halves of the position
    out = np.array(cache, copy=True)
    for b in range(len(start)):
        for j in range(int(cu[b + 1] - cu[b])):
            t = int(start[b]) + j
            if t >= pt.shape[1] * 64:
                continue
            out[pt[b, t % pt.shape[1]], t // pt.shape[1] % 64] = new[cu[b] + j]
    return out, scale


def _off_by_one(new, cu, start, cache, scale, kv_dtype, pt):
    return oracle.kv_append(new, cu, np.asarray(start) + 1, cache, scale, kv_dtype, pt)


def _first_request_table(new, cu, start, cache, scale, kv_dtype, pt):
    return oracle.kv_append(new, cu, start, cache, scale, kv_dtype, np.repeat(pt[:1], len(pt), axis=0))


@pytest.mark.parametrize("mutant", [_swapped, _off_by_one, _first_request_table], ids=lambda f: f.__name__)
def test_placement_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        _check_placement(mutant, "bf16")


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("page_size", [128, 1536])
def test_placement_any_page_size(kv_dtype, page_size):
    """A page of P rows is P / 64 consecutive 64-row pages: appending into a P-row cache
    equals appending into the same memory seen as 64-row pages through the expanded table."""
    rng = np.random.default_rng(71)
    k = page_size // 64
    batch, entries = 2, 3
    num_pages = batch * entries + 1
    pt = rng.permutation(num_pages)[: batch * entries].reshape(batch, entries).astype(np.int32)
    if kv_dtype == "bf16":
        cache = rng.integers(0, 1 << 16, size=(num_pages, page_size, 576), dtype=np.uint16)
        scale = None
    else:
        cache = rng.integers(-127, 128, size=(num_pages, page_size, 576), dtype=np.int8)
        if kv_dtype == "fp8":
            cache = cache.view(np.uint8)
        scale = rng.random((num_pages, page_size), dtype=np.float32)
    start = np.array([page_size - 5, 3], np.int32)
    n = np.array([70, 9], np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    new = synth.bf16_bits(rng.standard_normal((int(cu[-1]), 576)).astype(np.float32))
    big, big_sc = oracle.kv_append(new, cu, start, cache, scale, kv_dtype, pt)
    pt64 = (pt[:, :, None] * k + np.arange(k)[None, None, :]).reshape(batch, entries * k).astype(np.int32)
    small, small_sc = oracle.kv_append(new, cu, start, cache.reshape(num_pages * k, 64, 576),
                                       None if scale is None else scale.reshape(num_pages * k, 64), kv_dtype, pt64)
    assert np.array_equal(big.reshape(num_pages * k, 64, 576), small)
    if scale is not None:
        assert np.array_equal(big_sc.reshape(num_pages * k, 64), small_sc)
    assert not np.array_equal(big, cache)                 # something was written
