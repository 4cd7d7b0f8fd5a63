"""GPU-side helpers for the parity tests: move synth cases to the device and
call the library through its C ABI binding.  No arithmetic of the method here."""
import numpy as np
import torch

import mla_attention_paged_amd as mla

ATOL = 1e-2
RTOL = 1e-2
LSE_ATOL = 1e-3


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
    # diagnostic: relative Frobenius error per (token, head) row
    rel = np.linalg.norm(out - ref_out, axis=-1) / np.maximum(np.linalg.norm(ref_out, axis=-1), 1e-30)
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
