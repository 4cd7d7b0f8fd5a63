"""Oracle of the products on either side of the absorbed attention (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this module; the library's compute path never does.

What it follows.  [TALK] "构建面向 Agentic 推理的下一代 LLM 推理引擎", section
"Kernel：让 MLA 真正跑满 GPU": MLA compresses the KV of all heads into one latent
row per token, and decode's first product is query x latent key.  The absorbed
form that product takes, and the per-head up-projections, are the published MLA
formulation [MLA] (DeepSeek-V2, arXiv:2405.04434): per head h, the key's
no-position part is k_nope = W_UK[h] c and the value is v = W_UV[h] c for the
latent row c (512 values), with W_UK[h], W_UV[h] of shape [128, 512]; the query
is [q_nope (128); q_rope (64)] and the key [k_nope; k_rope (64)].  Hence

    q_nope . (W_UK[h] c) = (W_UK[h]^T q_nope) . c              (absorption)
    sum_t p_t W_UV[h] c_t = W_UV[h] (sum_t p_t c_t)            (up-projection)

so attention can run on the latent rows [c; k_rope] with the absorbed query
[W_UK[h]^T q_nope; q_rope], and the head output is W_UV[h] applied to the latent
output.  Everything here is float64 over exactly widened bf16 inputs; numpy's
einsum is the only primitive.
"""
from __future__ import annotations

import math

import numpy as np

D_NOPE = 128
D_ROPE = 64
D_LAT = 512
D_V = 128


def _f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def q_absorb(q_bits: np.ndarray, w_uk_bits: np.ndarray) -> np.ndarray:
    """Absorbed query [T, H, 576] = [W_UK[h]^T q_nope ; q_rope].

    q_bits: bf16 bits [T, H, 192] (q_nope 0..127 | q_rope 128..191);
    w_uk_bits: bf16 bits [H, 128, 512] (W_UK[h][d][c]).
    """
    q = _f64(q_bits)
    w = _f64(w_uk_bits)
    q_abs = np.einsum("hdc,thd->thc", w, q[..., :D_NOPE])
    return np.concatenate([q_abs, q[..., D_NOPE:]], axis=2)


def v_up(o: np.ndarray, w_uv_bits: np.ndarray) -> np.ndarray:
    """Head outputs [T, H, 128] = W_UV[h] o[t, h] for latent outputs o [T, H, 512]
    (float64, or bf16 bits when given as uint16); w_uv_bits: bf16 bits [H, 128, 512]."""
    o = _f64(o) if np.asarray(o).dtype == np.uint16 else np.asarray(o, dtype=np.float64)
    return np.einsum("hvc,thc->thv", _f64(w_uv_bits), o)


def mha_unabsorbed(q_bits, lat_bits, rope_bits, w_uk_bits, w_uv_bits, q_start, kv_len, softmax_scale):
    """Unabsorbed multi-head attention over per-request latent rows.

    q_bits: bf16 bits [T, H, 192]; lat_bits: list over requests of bf16 bits [L_b, 512]
    (latent rows c_t); rope_bits: list of bf16 bits [L_b, 64] (k_rope); q_start [B+1];
    kv_len [B].  Token i of request b (n_b tokens) sees rows 0 .. L_b - n_b + i.  Per head:
    k_t = [W_UK[h] c_t; k_rope_t], v_t = W_UV[h] c_t, out = softmax(scale q.k) v.
    Returns (out [T, H, 128], lse [T, H]) in float64.
    """
    q = _f64(q_bits)
    wk = _f64(w_uk_bits)
    wv = _f64(w_uv_bits)
    T, H, _ = q.shape
    out = np.zeros((T, H, D_V))
    lse = np.zeros((T, H))
    for b in range(len(kv_len)):
        c = _f64(lat_bits[b])
        kr = _f64(rope_bits[b])
        n = int(q_start[b + 1]) - int(q_start[b])
        L = int(kv_len[b])
        for h in range(H):
            k = np.concatenate([c @ wk[h].T, kr], axis=1)       # [L, 192]
            v = c @ wv[h].T                                     # [L, 128]
            for i in range(n):
                t = int(q_start[b]) + i
                vis = L - n + i + 1
                s = softmax_scale * (k[:vis] @ q[t, h])
                m = s.max()
                lse[t, h] = m + math.log(np.exp(s - m).sum())
                out[t, h] = (np.exp(s - lse[t, h])[:, None] * v[:vis]).sum(0)
    return out, lse
