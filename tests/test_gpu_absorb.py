"""Query absorption and value up-projection (GPU) against the oracle, and the whole
absorbed chain (absorb -> decode -> up-project, all on the GPU) against unabsorbed
multi-head attention ([MLA] per-head keys [W_UK c; k_rope] and values W_UV c)."""
import numpy as np
import pytest
import torch

import mla_attention_paged_amd as mla
import oracle
import synth
from mla_gpu import assert_close, dev_bf16, host, run_decode_varlen

pytestmark = pytest.mark.gpu

D_NOPE, D_ROPE, D_LAT, D_V = 128, 64, 512, 128


def _bits(x):
    return synth.bf16_bits(np.asarray(x, np.float32))


def _close(got, ref, what):
    """|got - ref| <= 1e-2 + 1e-2 |ref| elementwise (bf16 output of an fp32-accumulated product)."""
    err = np.abs(got - ref)
    bad = err > 1e-2 + 1e-2 * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements off, max err {err.max():.3g}"


def _absorb_gpu(q_bits, w_uk_bits):
    T, H, _ = q_bits.shape
    w_t = np.ascontiguousarray(np.transpose(w_uk_bits, (0, 2, 1)))         # [H, 512, 128]
    out = torch.empty((T, H, D_LAT + D_ROPE), dtype=torch.bfloat16, device="cuda")
    mla.mla_q_absorb(dev_bf16(q_bits), dev_bf16(w_t), out, T, H)
    return out


@pytest.mark.parametrize("T,H", [(1, 16), (16, 16), (64, 1), (65, 16), (129, 3), (130, 128), (3000, 16)])
def test_q_absorb_matches_oracle(T, H):
    rng = np.random.default_rng(800 + T)
    q = _bits(rng.standard_normal((T, H, D_NOPE + D_ROPE)))
    w = _bits(rng.standard_normal((H, D_NOPE, D_LAT)) * 0.05)
    out = _absorb_gpu(q, w)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.absorb.q_absorb(q, w)
    _close(got[..., :D_LAT], ref[..., :D_LAT], f"q_absorb {T}x{H}")
    assert np.array_equal(got[..., D_LAT:], ref[..., D_LAT:])            # the rope passes bit for bit


@pytest.mark.parametrize("T,H", [(1, 16), (16, 16), (64, 1), (65, 16), (129, 3), (130, 128), (3000, 16)])
def test_v_up_matches_oracle(T, H):
    rng = np.random.default_rng(900 + T)
    o = _bits(rng.standard_normal((T, H, D_LAT)))
    w = _bits(rng.standard_normal((H, D_V, D_LAT)) * 0.05)
    out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device="cuda")
    mla.mla_v_up(dev_bf16(o), dev_bf16(w), out, T, H)
    torch.cuda.synchronize()
    _close(out.float().cpu().numpy().astype(np.float64), oracle.absorb.v_up(o, w), f"v_up {T}x{H}")


def test_absorbed_chain_equals_unabsorbed_mha():
    """GPU: absorb the (nope | rope) queries, decode over the latent cache with ragged
    drafts, up-project; oracle: unabsorbed multi-head attention on the same rows."""
    rng = np.random.default_rng(1000)
    H, lens, drafts = 16, [700, 2000, 130], [2, 4, 1]
    lens = np.asarray(lens)
    case = synth.make_prefill_case(1001, H, prefix_lens=lens - np.asarray(drafts), new_lens=drafts)
    T = case.total_q()
    q_raw = _bits(rng.standard_normal((T, H, D_NOPE + D_ROPE)))
    w_uk = _bits(rng.standard_normal((H, D_NOPE, D_LAT)) * 0.05)
    w_uv = _bits(rng.standard_normal((H, D_V, D_LAT)) * 0.05)
    # GPU chain
    q_abs = _absorb_gpu(q_raw, w_uk)
    torch.cuda.synchronize()
    case.q = q_abs.view(torch.int16).cpu().numpy().view(np.uint16)      # the decode's input is the absorbed query
    o_lat, lse = run_decode_varlen(case, max_q_len=max(drafts))
    out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device="cuda")
    mla.mla_v_up(o_lat[:T].contiguous(), dev_bf16(w_uv), out, T, H)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    got_lse = lse[:T].cpu().numpy().astype(np.float64)
    # oracle: the logical rows of each request, split into latent and rope parts
    c = case.cache
    lat, rope = [], []
    for b in range(case.batch):
        rows = np.stack([c.data[c.page_table[b, t // 64], t % 64] for t in range(int(c.kv_lens[b]))])
        lat.append(rows[:, :D_LAT])
        rope.append(rows[:, D_LAT:])
    ref, ref_lse = oracle.absorb.mha_unabsorbed(q_raw, lat, rope, w_uk, w_uv, case.cu_seqlens_q, c.kv_lens,
                                                case.softmax_scale)
    _close(got, ref, "absorbed chain")
    assert np.abs(got_lse - ref_lse).max() <= 1e-3
