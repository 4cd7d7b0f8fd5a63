"""Decode, allocation-free decode, ragged decode, prefill and KV append captured into a
HIP graph (torch.cuda.CUDAGraph) and replayed (GPU).  The calls allocate nothing,
synchronise nothing and clear no memory with a memset, and their launch shapes depend
only on host scalars, so a captured call is replayed as is.  Every replay, with eager calls and synchronisations between replays,
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


def test_decode_noalloc_graph_replay():
    """The allocation-free decode, the entry point for callers that capture graphs."""
    import mla_attention_paged_amd as mla
    case = synth.make_decode_case(803, 3, 16, 2, seq_lens=[4000, 65, 1500])
    d = decode_inputs(case)
    out, lse, _ = _buffers(case, 1)

    def call(s):
        mla.mla_decode_noalloc(d["q"], d["kv"], d["scale"], d["kind"], d["pt"], case.cache.max_pages, d["seq_lens"],
                               case.batch, case.q_len, case.heads, case.cache.page_size, case.max_seq_len,
                               case.softmax_scale, out, lse, s)

    _replays_equal(call, out, lse)


def test_decode_varlen_graph_replay():
    import mla_attention_paged_amd as mla
    case = synth.make_prefill_case(804, 16, prefix_lens=[3000, 500, 64], new_lens=[1, 4, 2])
    d = prefill_inputs(case)
    T, H, mq = case.total_q(), case.heads, case.max_q_len()
    lens = torch.from_numpy(case.cache.kv_lens.copy()).cuda()
    out, lse, ws = _buffers(case, mla.mla_splitkv_workspace_size(case.batch, H, mq, T, case.max_seq_len, d["kind"]))

    def call(s):
        mla.mla_decode_varlen(d["q"], d["cu"], d["kv"], d["scale"], d["kind"], d["pt"], case.cache.max_pages, lens,
                              case.batch, T, mq, H, case.cache.page_size, case.max_seq_len, case.softmax_scale,
                              out, lse, ws, ws.numel(), s)

    _replays_equal(call, out, lse)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_append_graph_replay(kv_dtype):
    """mla_kv_append writes the same codes on every replay."""
    import mla_attention_paged_amd as mla
    rng = torch.Generator().manual_seed(805)
    rows, pages = 300, 8
    new = torch.randn((rows, 576), generator=rng).to(torch.bfloat16).cuda()
    cu = torch.tensor([0, 120, 120, 300], dtype=torch.int32, device="cuda")
    start = torch.tensor([10, 0, 100], dtype=torch.int32, device="cuda")
    pt = torch.randperm(pages * 3, generator=rng).to(torch.int32).reshape(3, pages).cuda()
    if kv_dtype == "bf16":
        kv = torch.zeros((pages * 3, 64, 576), dtype=torch.bfloat16, device="cuda")
        sc, kind = None, mla.MLA_KV_BF16
    else:
        kv = torch.zeros((pages * 3, 64, 576), dtype=torch.uint8, device="cuda")
        sc, kind = torch.zeros((pages * 3, 64), dtype=torch.float32, device="cuda"), mla.MLA_KV_FP8

    def call(s):
        mla.mla_kv_append(new, cu, start, kv, sc, kind, pt, pages, 3, rows, 64, s)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_kv, ref_sc = kv.clone(), (sc.clone() if sc is not None else None)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
    torch.cuda.synchronize()
    for _ in range(3):
        kv.zero_()
        if sc is not None:
            sc.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(kv.view(torch.uint8), ref_kv.view(torch.uint8))
        if sc is not None:
            assert torch.equal(sc, ref_sc)
