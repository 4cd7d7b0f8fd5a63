"""Every INT8 and FP8 code through the attention kernels (GPU).

A needle row holds all 256 byte values in its value columns (the two FP8 NaN bytes
replaced by +-448) with a power-of-two row scale; the query picks the needle's largest
code, so every other row's weight underflows to 0 in fp32 and each output row is the
needle's dequantised value columns, exact in bf16.  Needle b rotates the byte layout by
b, so over four needles every code sits at every byte position of a 32-bit word, and the
second half of a row is shifted by one more, so each needle shows each code twice.
The expected values decode the codes by their definition (two's complement bytes; E4M3
with bias 7, as the oracle decodes it)."""
import numpy as np
import pytest

import oracle
import synth
from mla_gpu import host, run_decode, run_prefill

pytestmark = pytest.mark.gpu

NEEDLE_SCALE = np.float32(0.5)
BF16_64 = int(synth.bf16_bits(np.array([64.0], np.float32))[0])


def _code_row(kv_dtype: str, r: int) -> np.ndarray:
    b = np.array([(k + r + k // 256) % 256 for k in range(512)], np.uint8)
    if kv_dtype == "fp8":
        b[b == 0x7F] = 0x7E
        b[b == 0xFF] = 0xFE
        return b
    return b.view(np.int8)


def _values(kv_dtype: str, codes: np.ndarray) -> np.ndarray:
    if kv_dtype == "int8":
        v = codes.astype(np.float32)
    else:
        v = np.array([oracle.e4m3_value(int(x)) for x in codes], np.float32)
    return v * NEEDLE_SCALE


def _plant(case, b: int, pos: int, r: int, rows):
    """Needle with rotation r at row `pos` of request b; the query rows `rows` select it."""
    c = case.cache
    page, slot = c.page_table[b, pos // c.page_size], pos % c.page_size
    codes = _code_row(c.kv_dtype, r)
    c.data[page, slot, :512] = codes
    c.scale[page, slot] = NEEDLE_SCALE
    vals = _values(c.kv_dtype, codes)
    j = int(np.argmax(vals))
    for t in rows:
        q = np.zeros((case.heads, 576), np.uint16)
        q[:, j] = BF16_64
        case.q[t] = q
    return synth.bf16_to_f32(synth.bf16_bits(vals))


def _check(out, rows, want, what):
    ok = out[rows] == want.astype(np.float64)[None, None, :]
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} values differ, first at {np.argwhere(~ok)[0]}"


def test_code_table_is_exhaustive():
    for r in range(4):
        assert sorted(set(_code_row("int8", r).view(np.uint8).tolist())) == list(range(256))
        fp8 = set(_code_row("fp8", r).tolist())
        assert fp8 == set(range(256)) - {0x7F, 0xFF}
        assert all(np.isfinite(_values("fp8", np.array(sorted(fp8), np.uint8))))


@pytest.mark.parametrize("kv_dtype", ["int8", "fp8"])
def test_decode_every_code_value(kv_dtype):
    seq = [5000, 700, 64, 9000]
    pos = [4998, 63, 0, 4096]
    case = synth.make_decode_case(701, batch=4, heads=16, q_len=2, seq_lens=seq, kv_dtype=kv_dtype)
    wants = [_plant(case, b, pos[b], b, range(2 * b, 2 * b + 2)) for b in range(4)]
    out, _ = host(*run_decode(case))
    for b in range(4):
        _check(out, list(range(2 * b, 2 * b + 2)), wants[b], f"{kv_dtype} decode needle {b} at row {pos[b]}")


@pytest.mark.parametrize("kv_dtype", ["int8", "fp8"])
def test_prefill_every_code_value(kv_dtype):
    prefix = [300, 0, 5000, 64]
    new = [5, 3, 70, 1]
    pos = [300, 0, 2500, 63]         # at or before each request's first new row: every new token sees it
    case = synth.make_prefill_case(702, 16, prefix_lens=prefix, new_lens=new, kv_dtype=kv_dtype)
    cu = case.cu_seqlens_q
    rows = [list(range(int(cu[b]), int(cu[b + 1]))) for b in range(4)]
    wants = [_plant(case, b, pos[b], b, rows[b]) for b in range(4)]
    out, _ = host(*run_prefill(case))
    for b in range(4):
        _check(out, rows[b], wants[b], f"{kv_dtype} prefill needle {b} at row {pos[b]}")
