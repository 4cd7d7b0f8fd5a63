"""mla_decode_noalloc (GPU): the allocation-free decode entry point against mla_decode on
the same inputs, two calls in a row (the second smaller, so that it runs on scratch the
first left dirty), plus its oversize rejection."""
import numpy as np
import pytest
import torch

import mla_attention_paged_amd as mla
import oracle
import synth
from mla_gpu import assert_close, bits, decode_inputs, host, run_decode

pytestmark = pytest.mark.gpu


def run_noalloc(case, d=None):
    d = d or decode_inputs(case)
    T, H = case.total_q(), case.heads
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    mla.mla_decode_noalloc(d["q"], d["kv"], d["scale"], d["kind"], d["pt"], case.cache.max_pages, d["seq_lens"],
                           case.batch, case.q_len, H, case.cache.page_size, case.max_seq_len, case.softmax_scale,
                           out, lse)
    return out, lse


def test_noalloc_matches_decode_two_calls():
    big = synth.make_decode_case(701, 4, 16, 4, seq_lens=[5000, 3000, 700, 64])
    small = synth.make_decode_case(702, 2, 16, 2, seq_lens=[300, 129])
    for case in (big, small):
        d = decode_inputs(case)
        ro, rl = run_decode(case, d)
        go, gl = run_noalloc(case, d)
        torch.cuda.synchronize()
        assert np.array_equal(bits(go), bits(ro)) and torch.equal(gl, rl), f"batch {case.batch}"
        o, l_ = host(go, gl)
        r, rlse = host(ro, rl)
        assert_close(o, l_, r, rlse, f"noalloc vs mla_decode, batch {case.batch}")
        ref_out, ref_lse = oracle.decode(case)
        assert_close(o, l_, ref_out, ref_lse, f"noalloc vs oracle, batch {case.batch}")


def test_noalloc_int8_and_single_workgroup():
    case = synth.make_decode_case(703, 3, 16, 2, seq_lens=[1500, 64, 777], kv_dtype="int8")
    d = decode_inputs(case)
    ro, rl = run_decode(case, d)
    go, gl = run_noalloc(case, d)
    assert np.array_equal(bits(go), bits(ro)) and torch.equal(gl, rl)
    one = synth.make_decode_case(704, 1, 16, 1, seq_lens=[40])  # one page: no split, no scratch
    d = decode_inputs(one)
    ro, rl = run_decode(one, d)
    go, gl = run_noalloc(one, d)
    assert np.array_equal(bits(go), bits(ro)) and torch.equal(gl, rl)


def test_noalloc_rejects_oversize_plan():
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_noalloc(t, t, None, 0, t, 4096, t, 4000, 4, 16, 64, 262144, 0.07, t, t)
    assert e.value.status == mla.MLA_ERR_SCRATCH
