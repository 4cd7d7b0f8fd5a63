"""Decode and prefill captured into a HIP graph (torch.cuda.CUDAGraph) and replayed
(GPU).  The calls allocate nothing, synchronise nothing and clear no memory with a
memset, and their launch shapes depend only on host scalars, so a captured call is
replayed as is.  Every replay, with eager calls and synchronisations between replays,
must equal the eager result bit for bit."""
import pytest
import torch

import synth
from mla_gpu import decode_inputs, prefill_inputs, run_decode, run_prefill

pytestmark = pytest.mark.gpu


def _replays_equal(call, out, lse, replays=3):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
    torch.cuda.synchronize()
    for _ in range(replays):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse, ref_l)
        call(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))


def _buffers(case, nbytes):
    T, H = max(case.total_q(), 1), case.heads
    return (torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda"),
            torch.empty((T, H), dtype=torch.float32, device="cuda"),
            torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_decode_graph_replay(kv_dtype):
    import mla_attention_paged_amd as mla
    case = synth.make_decode_case(801, 4, 16, 4, seq_lens=[5000, 300, 4096, 77], kv_dtype=kv_dtype)
    d = decode_inputs(case)
    out, lse, ws = _buffers(case, mla.mla_splitkv_workspace_size(
        case.batch, case.heads, case.q_len, case.total_q(), case.max_seq_len, d["kind"]))
    _replays_equal(lambda s: run_decode(case, d, out, lse, ws, s), out, lse)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prefill_graph_replay(kv_dtype):
    import mla_attention_paged_amd as mla
    case = synth.make_prefill_case(802, 16, prefix_lens=[3000, 0, 700], new_lens=[40, 9, 130],
                                   kv_dtype=kv_dtype)
    d = prefill_inputs(case)
    out, lse, ws = _buffers(case, mla.mla_splitkv_workspace_size(
        case.batch, case.heads, case.max_q_len(), case.total_q(), case.max_seq_len, d["kind"]))
    _replays_equal(lambda s: run_prefill(case, d, out, lse, ws, s), out, lse)
