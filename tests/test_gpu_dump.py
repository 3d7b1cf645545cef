"""attn_fwd_dump: the intermediates of one key tile of one prefill workgroup (logits S, P,
the running softmax's reference maximum m and running sum l) against the oracle's
logits for that block (flash-sparse-attention issue #11 page, "Next Steps": compare one
block's intermediate logits and mask values step by step)."""
import numpy as np
import pytest

import synth
from helpers import say, to_device

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


def block_logits(p, b, g, qb, qpb):
    """fp64 logits (scale q k^T + mask) of the workgroup's rows, rows query-major
    (r = (i - first) * G + h - g * G), and the number of valid rows."""
    import oracle
    G = p.Hq // p.Hkv
    q, k = p.f64("q"), p.f64("k")
    i0 = qb * qpb
    i1 = min(p.Lq, i0 + qpb)
    rows = (i1 - i0) * G
    A = oracle.mask_matrix(p.mask_kind, p.Lq, p.Lk, window_left=p.window_left,
                           dense=None if p.mask is None else p.mask.astype(np.float64))
    S = np.full((128, p.Lk), np.nan)
    for r in range(rows):
        i, h = i0 + r // G, g * G + r % G
        S[r] = p.scale64 * (k[b, g] @ q[b, h, i]) + A[i]
    return S, rows


@pytest.mark.parametrize("kind,tile,d", [("causal", 3, 128), ("causal", 4, 128), ("causal", 0, 128),
                                         ("window", 4, 128), ("dense", 2, 128), ("dense", 3, 64),
                                         ("none", 1, 128)])
def test_dump_matches_the_block_logits(kind, tile, d):
    import masked_flashattention_forward_amd as mfa
    B, Hq, Hkv, Lq, Lk = 2, 4, 2, 100, 300
    mask = synth.window_dense_mask(Lq, Lk, Lk - Lq, 90) if kind == "dense" else None
    p = synth.make_problem(f"dump {kind} d{d} tile {tile}", B, Hq, Hkv, Lq, Lk, d, "bf16", kind, 1700 + tile,
                           window_left=90, mask=mask)
    plan = mfa.plan(B, Hq, Hkv, Lq, Lk, d, kind, window_left=90)
    qpb = plan["block_m"] // (Hq // Hkv)
    b, g, qb = 1, 1, 1
    say(p.name)
    q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    import torch
    md = None if mask is None else torch.from_numpy(mask).cuda()
    out, lse, dump = mfa.attn_fwd_ex(q, k, v, scale=p.scale, mask_kind=kind, window_left=p.window_left, mask=md,
                                     dump_at=(b, g, qb, tile))
    torch.cuda.synchronize()
    S_ref, rows = block_logits(p, b, g, qb, qpb)
    j0 = 64 * tile
    nk = min(64, Lk - j0)
    S = dump["S"].cpu().numpy().astype(np.float64)
    P = dump["P"].cpu().numpy().astype(np.float64)
    m = dump["m"].cpu().numpy().astype(np.float64)
    l = dump["l"].cpu().numpy().astype(np.float64)
    # rows past the block are not written
    assert np.isnan(S[rows:]).all() and np.isnan(m[rows:]).all()
    Sr = S_ref[:rows, j0:j0 + nk]
    Sd = S[:rows, :nk]
    # masked entries are -inf exactly, visible ones the fp32 logits of the bf16 inputs
    np.testing.assert_array_equal(np.isneginf(Sd), np.isneginf(Sr))
    fin = np.isfinite(Sr)
    np.testing.assert_allclose(Sd[fin], Sr[fin], rtol=1e-5, atol=1e-4)
    # P = exp(S - m) with the dumped m
    with np.errstate(invalid="ignore"):
        ref_p = np.exp(Sd - m[:rows, None])
    ref_p[~fin] = 0.0
    np.testing.assert_allclose(P[:rows, :nk], ref_p, rtol=1e-5, atol=1e-30)
    # m trails the running maximum over the keys seen so far by less than 8 ln 2, and
    # l exp(m) is their partition sum
    seen = S_ref[:rows, :j0 + nk]
    with np.errstate(invalid="ignore"):
        run_max = np.max(np.where(np.isfinite(seen), seen, -np.inf), axis=1)
    live = np.isfinite(run_max)
    assert np.all(m[:rows][live] <= run_max[live] + 1e-4)
    assert np.all(m[:rows][live] >= run_max[live] - 8 * np.log(2) - 1e-4)
    z = np.exp(np.where(np.isfinite(seen), seen, -np.inf) - m[:rows, None]).sum(axis=1)
    np.testing.assert_allclose(l[:rows][live], z[live], rtol=1e-3)
    assert np.all(l[:rows][~live] == 0.0)
    print(f"[dump] {p.name}: {rows} rows, S/P/m/l consistent with the oracle logits", flush=True)


def test_dump_rejects_bad_requests():
    import torch
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem("dump errors", 1, 4, 2, 40, 300, 128, "bf16", "causal", 1710)
    q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    with pytest.raises(mfa.MiAttnError) as e:
        mfa.attn_fwd_ex(q, k, v, mask_kind="causal", dump_at=(0, 0, 0, 99))
    assert e.value.code == mfa.EINVAL
    # a decode-shaped call takes the split-KV decode kernel: no prefill workgroup to dump
    p2 = synth.make_problem("dump decode", 1, 4, 2, 1, 3000, 128, "bf16", "causal", 1711)
    q2, k2, v2 = (to_device(getattr(p2, n), p2.dtype) for n in ("q", "k", "v"))
    with pytest.raises(mfa.MiAttnError) as e:
        mfa.attn_fwd_ex(q2, k2, v2, mask_kind="causal", dump_at=(0, 0, 0, 0))
    assert e.value.code == mfa.EUNSUPPORTED
    # d = 64 with a position mask takes 128-key tiles: the 64-key dump refuses it
    p3 = synth.make_problem("dump d64 causal", 1, 4, 2, 200, 600, 64, "bf16", "causal", 1712)
    q3, k3, v3 = (to_device(getattr(p3, n), p3.dtype) for n in ("q", "k", "v"))
    with pytest.raises(mfa.MiAttnError) as e:
        mfa.attn_fwd_ex(q3, k3, v3, mask_kind="causal", dump_at=(0, 0, 0, 0))
    assert e.value.code == mfa.EUNSUPPORTED
    # score modifiers: the dump instances have none
    slopes = torch.full((p.Hq,), 0.25, dtype=torch.float32, device="cuda")
    for kw in (dict(alibi_slopes=slopes), dict(softcap=20.0)):
        with pytest.raises(mfa.MiAttnError) as e:
            mfa.attn_fwd_ex(q, k, v, mask_kind="causal", dump_at=(0, 0, 0, 0), **kw)
        assert e.value.code == mfa.EUNSUPPORTED
    torch.cuda.synchronize()


@pytest.mark.parametrize("keep,tile", [(100, 1), (400, 5)])
def test_dump_topk(keep, tile):
    """The top-k instances: with keep 100 the block's tiles are runs of its kept-key list
    (keys up to the block's last position whose rank is at most the first row's
    threshold, ascending, padded with key Lk); with keep 400 the list would not save
    enough and the tiles are consecutive keys. S holds scale q k^T + zero_hold on the keys
    a row keeps and -inf elsewhere (padding included), against the oracle's ranks and
    thresholds."""
    import torch
    import masked_flashattention_forward_amd as mfa
    from oracle.topk import topk_rank_ref, topk_tau_ref, kept_from_rank_tau
    B, Hq, Hkv, Lq, Lk, d = 1, 4, 2, 200, 600, 128
    G = Hq // Hkv
    p = synth.make_problem(f"dump top-k keep {keep} tile {tile}", B, Hq, Hkv, Lq, Lk, d, "bf16", "topk", 1720 + keep,
                           keep_k=keep, with_zero_hold=True)
    plan = mfa.plan(B, Hq, Hkv, Lq, Lk, d, "topk", keep_k=keep)
    gathered = plan["topk_list_cap"] > 0
    assert gathered == (keep == 100), plan
    qpb = plan["block_m"] // G
    b, g, qb = 0, 1, 2
    say(p.name)
    q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    zh = torch.from_numpy(p.zero_hold).cuda()
    out, lse, dump = mfa.attn_fwd_ex(q, k, v, scale=p.scale, mask_kind="topk", zero_hold=zh, keep_k=keep,
                                     dump_at=(b, g, qb, tile))
    torch.cuda.synchronize()
    zrow = p.zero_hold[b, g].astype(np.float64)
    rank = topk_rank_ref(zrow)
    tau = topk_tau_ref(rank, Lq, keep)
    kept = kept_from_rank_tau(rank, tau, Lq)
    i0, i1 = qb * qpb, min(Lq, qb * qpb + qpb)
    rows = (i1 - i0) * G
    pos_last = Lk - Lq + i1 - 1
    if gathered:
        keys = [j for j in range(pos_last + 1) if rank[j] <= tau[i0]]
        keys += [Lk] * (-len(keys) % 64)
    else:
        keys = list(range(Lk)) + [Lk] * (-Lk % 64)
    qf, kf = p.f64("q"), p.f64("k")
    S_all = np.full((rows, len(keys)), -np.inf)
    for r in range(rows):
        i, h = i0 + r // G, g * G + r % G
        for c, j in enumerate(keys):
            if j < Lk and kept[i, j]:
                S_all[r, c] = p.scale64 * (kf[b, g, j] @ qf[b, h, i]) + zrow[j]
    c0 = 64 * tile
    assert c0 < len(keys)
    Sr = S_all[:, c0:c0 + 64]
    S = dump["S"].cpu().numpy().astype(np.float64)[:rows]
    P = dump["P"].cpu().numpy().astype(np.float64)[:rows]
    m = dump["m"].cpu().numpy().astype(np.float64)[:rows]
    l = dump["l"].cpu().numpy().astype(np.float64)[:rows]
    np.testing.assert_array_equal(np.isneginf(S), np.isneginf(Sr))
    fin = np.isfinite(Sr)
    assert fin.any()
    np.testing.assert_allclose(S[fin], Sr[fin], rtol=1e-5, atol=1e-4)
    with np.errstate(invalid="ignore"):
        ref_p = np.exp(S - m[:, None])
    ref_p[~fin] = 0.0
    np.testing.assert_allclose(P, ref_p, rtol=1e-5, atol=1e-30)
    seen = S_all[:, :c0 + 64]
    run_max = np.max(seen, axis=1)
    live = np.isfinite(run_max)
    assert np.all(m[live] <= run_max[live] + 1e-4)
    assert np.all(m[live] >= run_max[live] - 8 * np.log(2) - 1e-4)
    z = np.exp(seen - m[:, None]).sum(axis=1)
    np.testing.assert_allclose(l[live], z[live], rtol=1e-3)
    print(f"[dump] {p.name}: {'kept-key list' if gathered else 'key'} tile {tile}, {rows} rows, "
          f"{int(fin.sum())} visible logits match the oracle", flush=True)
