"""GPU-side helpers for the parity tests: move synth cases to the device and
call the library through its C ABI binding.  No arithmetic of the method here."""
import numpy as np
import torch

import mla_attention_paged_amd as mla

ATOL = 1e-2
RTOL = 1e-2
LSE_ATOL = 1e-3
# Per (token, head) row: ||out - ref|| / ||ref|| over the 512 value columns.  The GPU path
# rounds three times to bf16 where the fp64 definition does not (the probabilities before
# the value product, the split-KV partials, the output), each a relative error of at most
# 2^-8 per element with an RMS of about 2^-8 / sqrt(3); over 512 columns the row ratio
# concentrates near their combined RMS, about 2^-8.  The bound is four times that.  It is
# what catches a wrong value path at long lengths, where |ref| ~ 0.02 and the elementwise
# absolute term alone would pass errors of half the value.
REL_FROB = 2.0 ** -6
# rows whose reference norm is below this are left to the elementwise bound
REL_FROB_MIN_NORM = 1e-3


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev_cache(cache, device="cuda"):
    if cache.kv_dtype == "bf16":
        data = dev_bf16(cache.data, device)
        scale = None
        kind = mla.MLA_KV_BF16
    else:
        data = torch.from_numpy(np.ascontiguousarray(cache.data)).to(device)
        scale = torch.from_numpy(np.ascontiguousarray(cache.scale)).to(device)
        kind = mla.MLA_KV_INT8 if cache.kv_dtype == "int8" else mla.MLA_KV_FP8
    pt = torch.from_numpy(np.ascontiguousarray(cache.page_table)).to(device)
    return data, scale, kind, pt


def decode_inputs(case, device="cuda"):
    data, scale, kind, pt = dev_cache(case.cache, device)
    return dict(q=dev_bf16(case.q, device), kv=data, scale=scale, kind=kind, pt=pt,
                seq_lens=torch.from_numpy(case.seq_lens.copy()).to(device))


def run_decode(case, inputs=None, out=None, lse=None, workspace=None, stream=None):
    d = inputs or decode_inputs(case)
    T, H = case.total_q(), case.heads
    out = out if out is not None else torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = lse if lse is not None else torch.empty((T, H), dtype=torch.float32, device="cuda")
    nbytes = mla.mla_splitkv_workspace_size(case.batch, H, case.q_len, T, case.max_seq_len, d["kind"])
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    mla.mla_decode(d["q"], d["kv"], d["scale"], d["kind"], d["pt"], case.cache.max_pages, d["seq_lens"],
                   case.batch, case.q_len, H, case.cache.page_size, case.max_seq_len, case.softmax_scale, out, lse, workspace,
                   workspace.numel(), stream)
    return out, lse


def prefill_inputs(case, device="cuda"):
    data, scale, kind, pt = dev_cache(case.cache, device)
    return dict(q=dev_bf16(case.q, device), kv=data, scale=scale, kind=kind, pt=pt,
                cu=torch.from_numpy(case.cu_seqlens_q.copy()).to(device),
                prefix=torch.from_numpy(case.prefix_lens.copy()).to(device))


def run_prefill(case, inputs=None, out=None, lse=None, workspace=None, stream=None):
    d = inputs or prefill_inputs(case)
    T, H = case.total_q(), case.heads
    out = out if out is not None else torch.empty((max(T, 1), H, 512), dtype=torch.bfloat16, device="cuda")
    lse = lse if lse is not None else torch.empty((max(T, 1), H), dtype=torch.float32, device="cuda")
    nbytes = mla.mla_splitkv_workspace_size(case.batch, H, case.max_q_len(), T, case.max_seq_len, d["kind"])
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    mla.mla_prefill_varlen(d["q"], d["cu"], d["prefix"], d["kv"], d["scale"], d["kind"], d["pt"],
                           case.cache.max_pages, case.batch, T, case.max_q_len(), case.max_seq_len, H,
                           case.cache.page_size,
                           case.softmax_scale, out, lse, workspace, workspace.numel(), stream)
    return out, lse


def host(out: torch.Tensor, lse: torch.Tensor):
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def assert_close(out, lse, ref_out, ref_lse, what=""):
    """|out - ref| <= 1e-2 + 1e-2 |ref| elementwise; |lse - ref| <= 1e-3."""
    assert out.shape == ref_out.shape, (out.shape, ref_out.shape)
    assert np.isfinite(out).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    err = np.abs(out - ref_out)
    bound = ATOL + RTOL * np.abs(ref_out)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (f"{what}: out mismatch at {worst}: got {out[worst]} ref {ref_out[worst]}"
                                  f" ({int((err > bound).sum())} elements out of tolerance)")
    lerr = np.abs(lse - ref_lse)
    assert (lerr <= LSE_ATOL).all(), f"{what}: lse max error {lerr.max()} at {np.argmax(lerr)}"
    # relative Frobenius error per (token, head) row
    rnorm = np.linalg.norm(ref_out, axis=-1)
    rel = np.linalg.norm(out - ref_out, axis=-1) / np.maximum(rnorm, 1e-30)
    rel = np.where(rnorm >= REL_FROB_MIN_NORM, rel, 0.0)
    worst_r = np.unravel_index(np.argmax(rel), rel.shape)
    assert rel.max() <= REL_FROB, (f"{what}: row {worst_r} relative Frobenius error {rel.max():.4g} "
                                   f"> {REL_FROB:.4g} ({int((rel > REL_FROB).sum())} rows)")
    print(f"[parity] {what}: max abs err {err.max():.3g}, lse err {lerr.max():.3g}, "
          f"row rel frob max {rel.max():.3g} mean {rel.mean():.3g}")
    return float(err.max()), float(lerr.max()), float(rel.max())


def run_decode_varlen(case, inputs=None, max_q_len=None, stream=None):
    """mla_decode_varlen on a PrefillCase read as a ragged decode (request b's n_b query
    tokens are the last n_b of its seq_lens[b] cached rows)."""
    d = inputs or prefill_inputs(case)
    T, H = case.total_q(), case.heads
    mq = max_q_len or max(1, case.max_q_len())
    out = torch.empty((max(T, 1), H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((max(T, 1), H), dtype=torch.float32, device="cuda")
    lens = torch.from_numpy(case.cache.kv_lens.copy()).cuda()
    nbytes = mla.mla_splitkv_workspace_size(case.batch, H, mq, T, case.max_seq_len, d["kind"])
    workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    mla.mla_decode_varlen(d["q"], d["cu"], d["kv"], d["scale"], d["kind"], d["pt"], case.cache.max_pages, lens,
                          case.batch, T, mq, H, case.cache.page_size, case.max_seq_len, case.softmax_scale, out,
                          lse, workspace,
                          workspace.numel(), stream)
    return out, lse


def sample_prefill_tokens(case, tok_per_tile: int, rate: float = 1.0 / 32, seed: int = 0):
    """Query tokens whose rows a sampled parity check compares: the first and last new token
    of every request, plus one seeded token from each of a seeded ``rate`` share of the work
    tiles (``tok_per_tile`` consecutive new tokens of one request), so that tiles in the
    middle of long requests are covered too.  Returns sorted global token indices."""
    g = np.random.default_rng(seed)
    cu = case.cu_seqlens_q
    toks = set()
    for b in range(case.batch):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        toks.update((lo, hi - 1))
        ntiles = (hi - lo + tok_per_tile - 1) // tok_per_tile
        for t in np.nonzero(g.random(ntiles) < rate)[0]:
            j0 = lo + int(t) * tok_per_tile
            toks.add(int(g.integers(j0, min(hi, j0 + tok_per_tile))))
    return sorted(toks)


def permute_pages(cache, seed: int):
    """The same logical rows at new physical pages (data, scales and page table moved together)."""
    perm = np.random.default_rng(seed).permutation(cache.num_pages)
    nd = np.empty_like(cache.data)
    nd[perm] = cache.data
    cache.data = nd
    if cache.scale is not None:
        ns = np.empty_like(cache.scale)
        ns[perm] = cache.scale
        cache.scale = ns
    cache.page_table = perm[cache.page_table].astype(np.int32)
    cache.poison_page = int(perm[cache.poison_page])
    return cache


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor."""
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)
