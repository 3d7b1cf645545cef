"""Rows past the key count read nothing: each path gets K/V whose memory just past the last
key (inside the allocation) holds NaN, and must still match the oracle with no NaN
anywhere. A tile that reaches past Lk relies on the buffer range check (direct loads),
on clamped indices (varlen, paged) or on the per-row bounds of the fp32 kernel; finite
garbage there would be masked and multiplied by P = 0 and go unseen, NaN does not
(ExecuTorch pull request #10466 page, "Summary": the -inf tail of a chunk must not turn
into NaN; flash-sparse-attention issue #11 page, "Suspected Issues": index and off-by-one
errors)."""
import numpy as np
import pytest

import synth
from helpers import compare, out_to_f64, run_oracle, run_oracle_paged, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_flashattention_forward_amd as mfa
    mfa.lib()
    mfa.set_debug()
    yield
    mfa.set_debug()


def padded(t, pad):
    """The same values as a view of a [B, H, L + pad, d] allocation whose rows L.. are NaN."""
    import torch
    B, H, L, d = t.shape
    buf = torch.full((B, H, L + pad, d), float("nan"), dtype=t.dtype, device=t.device)
    buf[:, :, :L] = t
    return buf[:, :, :L]


def run_padded(p, pad=96, path=None, splits=0):
    import torch
    import masked_flashattention_forward_amd as mfa
    q = to_device(p.q, p.dtype)
    k = padded(to_device(p.k, p.dtype), pad)
    v = padded(to_device(p.v, p.dtype), pad)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((p.B, p.Hq, p.Lq), float("nan"), dtype=torch.float32, device="cuda")
    zh = None if p.zero_hold is None else torch.from_numpy(p.zero_hold).cuda()
    mask = None if p.mask is None else torch.from_numpy(p.mask).cuda()
    mfa.set_debug(force_path=-1 if path is None else path, force_splits=splits)
    try:
        mfa.attn_fwd_ex(q, k, v, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left,
                        mask=mask if p.mask_kind == "dense" else None, zero_hold=zh, keep_k=p.keep_k,
                        out=out, lse=lse)
        torch.cuda.synchronize()
    finally:
        mfa.set_debug()
    return out_to_f64(out, p.dtype), lse.cpu().numpy().astype(np.float64)


def check_padded(p, label, **kw):
    say(label)
    out, lse = run_padded(p, **kw)
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=label)


@pytest.mark.parametrize("kind", ["none", "causal", "window", "dense", "topk"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
def test_prefill_path_nan_past_lk(kind, dtype, d):
    """MFMA prefill kernel (path 1), ragged last tile (203 keys = 3 tiles + 11)."""
    Lq, Lk = 77, 203
    mask = synth.window_dense_mask(Lq, Lk, Lk - Lq, 150) if kind == "dense" else None
    p = synth.make_problem(f"poison prefill {kind} {dtype} d{d}", 2, 4, 2, Lq, Lk, d, dtype, kind, 1300 + d,
                           window_left=50, keep_k=40, with_zero_hold=kind == "topk", mask=mask)
    check_padded(p, p.name, path=1)
    check_padded(p, p.name + " split 3", path=1, splits=3)


def test_gathered_topk_nan_past_lk():
    """Top-k over kept-key lists: the list padding entries carry key index Lk, so every
    padded row of a gathered tile points at the first NaN row."""
    import masked_flashattention_forward_amd as mfa
    B, Hq, Hkv, Lq, Lk, keep = 1, 4, 2, 700, 1013, 100
    assert mfa.plan(B, Hq, Hkv, Lq, Lk, 128, "topk", keep_k=keep)["topk_list_cap"] > 0
    p = synth.make_problem("poison gathered top-k", B, Hq, Hkv, Lq, Lk, 128, "bf16", "topk", 1310, keep_k=keep,
                           with_zero_hold=True)
    check_padded(p, p.name)


@pytest.mark.parametrize("G,Lq,Lk", [(4, 1, 1500), (8, 4, 777), (1, 1, 33)])
def test_decode_path_nan_past_lk(G, Lq, Lk):
    """Split-KV decode kernel (path 2): 32-key tiles, ragged ends."""
    p = synth.make_problem(f"poison decode G{G} Lq{Lq} Lk{Lk}", 2, 2 * G, 2, Lq, Lk, 128, "bf16", "causal", 1320 + Lk)
    check_padded(p, p.name, path=2)
    check_padded(p, p.name + " split 5", path=2, splits=5)


@pytest.mark.parametrize("kind", ["causal", "none", "dense"])
def test_row_path_nan_past_lk(kind):
    """fp32 row kernel (path 0)."""
    Lq, Lk = 33, 90
    mask = synth.window_dense_mask(Lq, Lk, Lk - Lq, 20) if kind == "dense" else None
    p = synth.make_problem(f"poison row {kind}", 2, 4, 2, Lq, Lk, 64, "fp32", kind, 1330, mask=mask)
    check_padded(p, p.name, path=0)


def test_contiguous_attn_fwd_nan_after_last_head():
    """attn_fwd on contiguous K/V whose allocation continues with NaN after the last key of
    the last (batch, head): the tiles of that head reach past the end of its rows."""
    import torch
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem("poison contiguous tail", 2, 8, 2, 130, 333, 128, "bf16", "causal", 1340)
    say(p.name)

    def tail(a):
        t = to_device(a, p.dtype)
        buf = torch.full((t.numel() + 64 * p.d,), float("nan"), dtype=t.dtype, device="cuda")
        buf[:t.numel()] = t.flatten()
        return buf[:t.numel()].view(t.shape)

    q, k, v = to_device(p.q, p.dtype), tail(p.k), tail(p.v)
    out, lse = mfa.attn_fwd(q, k, v, scale=p.scale, mask_kind="causal")
    torch.cuda.synchronize()
    ref_o, ref_l = run_oracle(p)
    compare(p, out_to_f64(out, p.dtype), lse.cpu().numpy().astype(np.float64), ref_o, ref_l, label=p.name)


# ------------------------------------------------------------------ varlen / paged
def run_varlen_poisoned(p, extra_rows=0, kv_rows=None, cu_k=None):
    """attn_fwd_varlen with the K/V storage poisoned where no sequence has a key: the
    slots of each sequence's last page past its cached keys and the spare pages (paged),
    or extra NaN rows after the last sequence (packed). ``kv_rows`` (packed) passes only
    the first kv_rows rows of the allocation; ``cu_k`` overrides the key offsets."""
    import torch
    import masked_flashattention_forward_amd as mfa
    q = to_device(p.q, p.dtype)
    k, v = to_device(p.k, p.dtype), to_device(p.v, p.dtype)
    k_lens = np.diff(p.cu_seqlens_k)
    q_lens = np.diff(p.cu_seqlens_q)
    if p.block_table is not None:
        used = np.zeros(k.shape[:2], dtype=bool)
        cached = np.maximum(k_lens - q_lens, 0) if p.two_source else k_lens
        for s, n in enumerate(cached.tolist()):
            j = np.arange(n)
            used[p.block_table[s][j // p.page_size], j % p.page_size] = True
        bad = torch.from_numpy(~used).cuda()
        k[bad] = float("nan")
        v[bad] = float("nan")
    else:
        if extra_rows:
            pad = torch.full((extra_rows,) + tuple(k.shape[1:]), float("nan"), dtype=k.dtype, device="cuda")
            k, v = torch.cat([k, pad]), torch.cat([v, pad.clone()])
        if kv_rows is not None:
            k[kv_rows:] = float("nan")
            v[kv_rows:] = float("nan")
            k, v = k[:kv_rows], v[:kv_rows]
    kn = vn = None
    if p.two_source:
        kn, vn = to_device(p.k_new, p.dtype), to_device(p.v_new, p.dtype)
    cu_q = torch.from_numpy(p.cu_seqlens_q).cuda()
    cu_k_t = torch.from_numpy(p.cu_seqlens_k if cu_k is None else np.asarray(cu_k, dtype=np.int32)).cuda()
    bt = None if p.block_table is None else torch.from_numpy(p.block_table).cuda()
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((p.total_q, p.Hq), float("nan"), dtype=torch.float32, device="cuda")
    mk = int(np.diff(cu_k_t.cpu().numpy()).max())
    mfa.attn_fwd_varlen(q, k, v, cu_q, cu_k_t, max_seqlen_q=p.max_seqlen_q, max_seqlen_k=mk, block_table=bt,
                        k_new=kn, v_new=vn, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left,
                        out=out, lse=lse)
    torch.cuda.synchronize()
    return out_to_f64(out, p.dtype), lse.cpu().numpy().astype(np.float64)


Q_LENS = [1, 37, 1, 130, 0, 5, 70]
K_LENS = [300, 200, 1, 130, 50, 3, 201]


@pytest.mark.parametrize("page_size,two", [(16, False), (128, False), (16, True), (0, False), (0, True)])
@pytest.mark.parametrize("kind", ["causal", "none"])
def test_varlen_nan_in_unused_storage(page_size, two, kind):
    p = synth.make_paged_problem(f"poison varlen page{page_size} two{int(two)} {kind}", Q_LENS, K_LENS, 8, 2, 128,
                                 "bf16", kind, 1350 + page_size, page_size=page_size, two_source=two)
    say(p.name)
    out, lse = run_varlen_poisoned(p, extra_rows=80)
    ref_o, ref_l = run_oracle_paged(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


def test_varlen_packed_lengths_past_kv_rows_stay_inside():
    """Invalid packed lengths: the last sequence's keys run 56 rows past the kv_rows rows
    passed (the view ends there; the allocation continues with NaN). Every index is
    clamped into the kv_rows rows, so that sequence's rows are finite (their values are
    unspecified) and the valid sequence still matches the oracle."""
    q_lens, k_lens = [40, 64], [100, 256]
    p = synth.make_paged_problem("poison varlen lengths past kv_rows", q_lens, k_lens, 8, 2, 128, "bf16",
                                 "causal", 1360, page_size=0)
    say(p.name)
    kv_rows = 300  # the second sequence claims rows 100..355
    out, lse = run_varlen_poisoned(p, extra_rows=0, kv_rows=kv_rows)
    assert not np.isnan(out).any() and not np.isnan(lse).any(), "a read left the kv_rows rows passed"
    ref_o, ref_l = run_oracle_paged(p, seqs=[0])
    compare(p, out, lse, ref_o, ref_l, rows=slice(None), label=p.name + " (valid sequence)")
