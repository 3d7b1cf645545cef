"""Shared test helpers: move a synthetic problem to the GPU, run the HIP path through the
binding, run the oracle on the same stored inputs, and compare to the stated bounds."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

# Bounds: fp32 inputs 1e-5 on the output; fp16/bf16 inputs 2e-2 on the output and 1e-3
# on the LSE; an LSE of -inf must match exactly and no NaN may appear.
TOL = {"fp32": (1e-5, 1e-5), "fp16": (2e-2, 1e-3), "bf16": (2e-2, 1e-3)}


def say(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def out_to_f64(t, dtype: str) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(p: synth.Problem, *, out_fill=None, return_tensors=False):
    import torch
    import masked_flashattention_forward_amd as mfa
    q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    mask = None if p.mask is None else torch.from_numpy(p.mask).cuda()
    zh = None if p.zero_hold is None else torch.from_numpy(p.zero_hold).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((p.B, p.Hq, p.Lq), dtype=torch.float32, device=q.device)
    if out_fill is not None:
        out.fill_(out_fill)
        lse.fill_(out_fill)
    mfa.attn_fwd(q, k, v, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left,
                 mask=mask if p.mask_kind == "dense" else None,
                 zero_hold=zh if p.mask_kind == "topk" else None,
                 keep_k=p.keep_k, out=out, lse=lse)
    torch.cuda.synchronize()
    if return_tensors:
        return out, lse
    return out_to_f64(out, p.dtype), lse.cpu().numpy().astype(np.float64)


def run_oracle(p: synth.Problem, rows=None, heads=None):
    return oracle.attention_ref(p.f64("q"), p.f64("k"), p.f64("v"), p.scale64, p.mask_kind,
                                window_left=p.window_left,
                                mask=None if p.mask is None else p.mask.astype(np.float64),
                                zero_hold=None if p.zero_hold is None else p.zero_hold.astype(np.float64),
                                keep_k=p.keep_k, rows=rows, heads=heads)


def compare(p: synth.Problem, out, lse, ref_out, ref_lse, rows=None, heads=None, label="", tol=None):
    """Element-wise comparison on the computed (rows, heads) subset; returns the errors.
    ``tol`` = (output, LSE) overrides the dtype's tolerances where a case derives its own."""
    tol_o, tol_l = TOL[p.dtype] if tol is None else tol
    sel = ~np.isnan(ref_lse)
    if rows is not None or heads is not None:
        assert sel.any()
    go, gl = out[sel], lse[sel]
    ro, rl = ref_out[sel], ref_lse[sel]
    # per-row tolerances (arrays shaped like the LSE) or one number for every row
    to = np.broadcast_to(np.asarray(tol_o, dtype=np.float64), ref_lse.shape)[sel]
    tl = np.broadcast_to(np.asarray(tol_l, dtype=np.float64), ref_lse.shape)[sel]
    assert not np.isnan(go).any(), f"{label}: NaN in output"
    assert not np.isnan(gl).any(), f"{label}: NaN in LSE"
    dead = rl == -np.inf
    assert np.array_equal(gl == -np.inf, dead), f"{label}: -inf LSE pattern differs"
    assert np.all(go[dead] == 0.0), f"{label}: fully masked rows must be 0"
    row_o = np.abs(go - ro).reshape(go.shape[0], -1).max(axis=1) if go.size else np.zeros(0)
    row_l = np.where(dead, 0.0, np.abs(gl - np.where(dead, 0.0, rl)))
    err_o = float(row_o.max()) if row_o.size else 0.0
    err_l = float(row_l.max()) if row_l.size else 0.0
    ratio_o = float((row_o / to).max()) if row_o.size else 0.0
    ratio_l = float((row_l / tl).max()) if row_l.size else 0.0
    print(f"[parity] {label or p.name}: max|out err|={err_o:.3e} (tol {float(to.min()):.3g}..{float(to.max()):.3g}) "
          f"max|lse err|={err_l:.3e} (tol {float(tl.min()):.3g}..{float(tl.max()):.3g}) "
          f"worst err/tol out {ratio_o:.3f} lse {ratio_l:.3f} dead_rows={int(dead.sum())}", flush=True)
    assert ratio_o <= 1.0, f"{label}: output error {err_o} exceeds its row's tolerance (worst ratio {ratio_o})"
    assert ratio_l <= 1.0, f"{label}: LSE error {err_l} exceeds its row's tolerance (worst ratio {ratio_l})"
    return err_o, err_l


# ---------------------------------------------------------------- varlen / paged problems
def run_gpu_paged(p: synth.PagedProblem, *, out_fill=None, max_seqlen_k=None, alibi=None, softcap=0.0):
    import torch
    import masked_flashattention_forward_amd as mfa
    q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    kn = vn = None
    if p.two_source:
        kn, vn = to_device(p.k_new, p.dtype), to_device(p.v_new, p.dtype)
    cu_q = torch.from_numpy(p.cu_seqlens_q).cuda()
    cu_k = torch.from_numpy(p.cu_seqlens_k).cuda()
    bt = None if p.block_table is None else torch.from_numpy(p.block_table).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((p.total_q, p.Hq), dtype=torch.float32, device=q.device)
    if out_fill is not None:
        out.fill_(out_fill)
        lse.fill_(out_fill)
    sl = None if alibi is None else torch.from_numpy(np.asarray(alibi, dtype=np.float32)).cuda()
    mfa.attn_fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q=p.max_seqlen_q,
                        max_seqlen_k=p.max_seqlen_k if max_seqlen_k is None else max_seqlen_k,
                        block_table=bt, k_new=kn, v_new=vn, scale=p.scale, mask_kind=p.mask_kind,
                        window_left=p.window_left, alibi_slopes=sl, softcap=softcap, out=out, lse=lse)
    torch.cuda.synchronize()
    return out_to_f64(out, p.dtype), lse.cpu().numpy().astype(np.float64)


def run_oracle_paged(p: synth.PagedProblem, seqs=None, alibi=None, softcap=0.0):
    """fp64 oracle; with ``seqs`` only those sequences are computed (their K/V rows are
    gathered from the cache in storage form first) and the other rows are NaN. ``alibi``
    (fp32 slopes) and ``softcap`` as passed to the GPU call."""
    mods = dict(alibi_slopes=None if alibi is None else np.asarray(alibi, dtype=np.float32).astype(np.float64),
                softcap=float(np.float32(softcap)))
    if seqs is None:
        return oracle.paged_attention_ref(p.f64("q"), p.f64("k"), p.f64("v"), p.cu_seqlens_q, p.cu_seqlens_k,
                                          p.block_table, p.page_size, p.scale, p.mask_kind,
                                          window_left=p.window_left, k_new=p.f64("k_new"), v_new=p.f64("v_new"),
                                          **mods)
    out = np.full((p.total_q, p.Hq, p.d), np.nan)
    lse = np.full((p.total_q, p.Hq), np.nan)
    for s in seqs:
        q0, q1 = int(p.cu_seqlens_q[s]), int(p.cu_seqlens_q[s + 1])
        Lk = int(p.k_lens[s])
        ctx = max(Lk - (q1 - q0), 0) if p.two_source else Lk
        j = np.arange(ctx)
        if p.block_table is None:
            rows_k = p.k[int(p.cu_seqlens_k[s]) + j]
            rows_v = p.v[int(p.cu_seqlens_k[s]) + j]
        else:
            pg = p.block_table[s][j // p.page_size]
            rows_k, rows_v = p.k[pg, j % p.page_size], p.v[pg, j % p.page_size]
        # a one-sequence packed problem holding all Lk rows (the new-token rows unused)
        kk = np.zeros((Lk,) + rows_k.shape[1:], dtype=rows_k.dtype)
        vv = np.zeros_like(kk)
        kk[:ctx], vv[:ctx] = rows_k, rows_v
        f = lambda a: synth.storage_to_f64(a, p.dtype)  # noqa: E731
        o, l = oracle.paged_attention_ref(
            f(p.q[q0:q1]), f(kk), f(vv), [0, q1 - q0], [0, Lk], None, 0, p.scale, p.mask_kind,
            window_left=p.window_left,
            k_new=None if not p.two_source else f(p.k_new[q0:q1]),
            v_new=None if not p.two_source else f(p.v_new[q0:q1]), **mods)
        out[q0:q1], lse[q0:q1] = o, l
    return out, lse
