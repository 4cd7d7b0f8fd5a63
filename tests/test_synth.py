"""The seeded input generator: rounding, determinism, paging and poison layout (CPU)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_lengths_are_seeded():
    c2 = synth.make_decode_case(3, 16, 32, 2, len_range=(32768, 131072))
    assert c2.seq_lens.tolist()[:4] == [112542, 41187, 50407, 56047]
    g = np.random.default_rng(4)
    P = g.integers(16384, 98304, size=8, endpoint=True)
    assert P.tolist()[0] == 75894


def test_same_seed_same_bytes_and_paging_layout():
    a = synth.make_decode_case(9, batch=3, heads=2, q_len=2, seq_lens=[130, 64, 7], max_seq_len=200)
    b = synth.make_decode_case(9, batch=3, heads=2, q_len=2, seq_lens=[130, 64, 7], max_seq_len=200)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.cache.data, b.cache.data)
    c = a.cache
    assert c.page_table.shape == (3, 4)
    used = [3, 1, 1]
    seen = set()
    for bi in range(3):
        for j in range(4):
            p = int(c.page_table[bi, j])
            if j < used[bi]:
                assert p != c.poison_page and p not in seen
                seen.add(p)
            else:
                assert p == c.poison_page
    assert len(seen) + 1 == c.num_pages
    poison = synth.bf16_bits(np.array([1000.0], np.float32))[0]
    # tails past each length in the last page hold the poison value
    assert (c.data[c.page_table[0, 2], 2:] == poison).all()
    assert not (c.data[c.page_table[0, 2], :2] == poison).all()
    assert (c.data[c.page_table[2, 0], 7:] == poison).all()
    assert (c.data[c.poison_page] == poison).all()


def test_int8_quantisation_rules():
    g = np.random.default_rng(1)
    x = g.standard_normal((50, 576)).astype(np.float32)
    codes, scale = synth.quantize_int8_rows(x)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    assert np.abs(codes).max() <= 127
    assert (np.abs(codes).max(axis=1) == 127).all()
    err = np.abs(codes.astype(np.float64) * scale[:, None] - x)
    assert (err <= scale[:, None] * 0.5 + 1e-6).all()


def test_prefill_case_layout():
    p = synth.make_prefill_case(5, heads=4, prefix_lens=[10, 0], new_lens=[3, 70])
    assert p.cu_seqlens_q.tolist() == [0, 3, 73]
    assert p.cache.kv_lens.tolist() == [13, 70]
    assert p.q.shape == (73, 4, 576)
    assert p.max_q_len() == 70
