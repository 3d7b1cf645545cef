"""Pins for the fp64 oracle, checked against facts fixed outside the oracle:
closed forms, invariants, a library routine (torch's CPU scaled-dot-product
attention in fp64), brute force, a second algorithm, and the worked cases the
pages describe (fixtures under tests/golden/). No GPU is used here."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (NEG_INF, attention_chunked_ref, attention_ref, attention_rows_ref,
                    kept_from_rank_tau, lse_merge_ref, mask_matrix, pack_keep_bits,
                    query_positions, topk_kept_ref, topk_rank_ref, topk_tau_ref)
from oracle.topk import INT32_MAX

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def torch_sdpa(q, k, v, scale, A=None, causal=False):
    """torch CPU fp64 attention (library routine), GQA via enable_gqa."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    am = None if A is None else torch.from_numpy(np.ascontiguousarray(A))
    G = q.shape[1] // k.shape[1]
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, is_causal=causal, scale=scale,
                                       enable_gqa=G > 1)
    return o.numpy()


# ---------------------------------------------------------------- softmax / PV closed forms
def test_single_visible_key_returns_its_v_row():
    Lq, Lk, d = 9, 23, 16
    q, k, v = rnd(1, Lq, d), rnd(2, Lk, d), rnd(3, Lk, d)
    A = mask_matrix("window", Lq, Lk, window_left=0)      # exactly key p_i
    out, lse = attention_rows_ref(q, k, v, 0.3, A)
    pos = query_positions(Lq, Lk)
    np.testing.assert_array_equal(out, v[pos])
    np.testing.assert_allclose(lse, 0.3 * np.einsum("id,id->i", q, k[pos]), rtol=0, atol=1e-15)


def test_constant_v_returns_the_constant():
    Lq, Lk, d = 7, 40, 8
    q, k = rnd(4, Lq, d), rnd(5, Lk, d)
    c = rnd(6, d)
    v = np.tile(c, (Lk, 1))
    for kind in ("none", "causal", "window"):
        out, _ = attention_rows_ref(q, k, v, 0.5, mask_matrix(kind, Lq, Lk, window_left=3))
        np.testing.assert_allclose(out, np.tile(c, (Lq, 1)), rtol=0, atol=1e-14)


def test_uniform_logits_give_mean_and_log_count():
    """K = 0 makes every visible logit equal: out is the plain mean of the visible V rows
    and LSE = ln(#visible) plus the mask constant (natural log, not log2)."""
    Lq, Lk, d = 6, 30, 4
    q, k, v = rnd(7, Lq, d), np.zeros((Lk, d)), rnd(8, Lk, d)
    A = mask_matrix("window", Lq, Lk, window_left=5)
    const = 1.75
    out, lse = attention_rows_ref(q, k, v, 1.0, A + const)
    pos = query_positions(Lq, Lk)
    for i in range(Lq):
        vis = np.arange(max(0, pos[i] - 5), pos[i] + 1)
        np.testing.assert_allclose(out[i], v[vis].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i] - (np.log(vis.size) + const)) < 1e-14


def test_output_lies_in_hull_of_visible_values():
    Lq, Lk, d = 12, 50, 8
    q, k, v = 3 * rnd(9, Lq, d), rnd(10, Lk, d), rnd(11, Lk, d)
    A = mask_matrix("causal", Lq, Lk)
    out, _ = attention_rows_ref(q, k, v, 1.0, A)
    pos = query_positions(Lq, Lk)
    for i in range(Lq):
        vis = v[: pos[i] + 1]
        assert np.all(out[i] >= vis.min(axis=0) - 1e-12) and np.all(out[i] <= vis.max(axis=0) + 1e-12)


def test_mask_shift_moves_lse_only():
    Lq, Lk, d = 5, 33, 8
    q, k, v = rnd(12, Lq, d), rnd(13, Lk, d), rnd(14, Lk, d)
    A = rnd(15, Lq, Lk)
    A[:, ::3] = NEG_INF
    c = np.array([0.5, -2.0, 3.0, 0.0, 10.0])[:, None]
    o1, l1 = attention_rows_ref(q, k, v, 0.7, A)
    o2, l2 = attention_rows_ref(q, k, v, 0.7, A + c)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, c[:, 0], rtol=0, atol=1e-13)


def test_lse_normalises_the_weights():
    """exp(z - lse) sums to one over a row and reproduces the output."""
    Lq, Lk, d = 8, 29, 4
    q, k, v = rnd(16, Lq, d), rnd(17, Lk, d), rnd(18, Lk, d)
    A = mask_matrix("causal", Lq, Lk)
    out, lse = attention_rows_ref(q, k, v, 0.9, A)
    with np.errstate(invalid="ignore"):
        w = np.exp(0.9 * q @ k.T + A - lse[:, None])
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(w @ v, out, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- guard / fully masked rows
def test_fully_masked_rows_return_zero_and_neg_inf():
    Lq, Lk, d = 4, 20, 8
    q, k, v = rnd(19, Lq, d), rnd(20, Lk, d), rnd(21, Lk, d)
    A = np.full((Lq, Lk), NEG_INF)
    A[1, 3] = 0.25
    out, lse = attention_rows_ref(q, k, v, 1.0, A)
    for i in (0, 2, 3):
        assert np.all(out[i] == 0.0) and lse[i] == NEG_INF
    np.testing.assert_array_equal(out[1], v[3])
    assert not np.isnan(out).any() and not np.isnan(lse).any()


def test_more_queries_than_keys_masks_leading_rows():
    Lq, Lk, d = 10, 6, 4
    q, k, v = rnd(22, 1, 1, Lq, d), rnd(23, 1, 1, Lk, d), rnd(24, 1, 1, Lk, d)
    out, lse = attention_ref(q, k, v, 1.0, "causal")
    assert np.all(out[0, 0, :4] == 0.0) and np.all(lse[0, 0, :4] == NEG_INF)
    np.testing.assert_array_equal(out[0, 0, 4], v[0, 0, 0])     # p_4 = 0 sees only key 0


@pytest.mark.parametrize("kind", ["none", "causal", "window", "dense", "topk"])
@pytest.mark.parametrize("chunk", [1, 7, 64, 128, 512])
def test_chunked_online_softmax_matches_plain_route(kind, chunk):
    Lq, Lk, d = 13, 300, 16
    q, k, v = rnd(25, Lq, d), rnd(26, Lk, d), rnd(27, Lk, d)
    zh = rnd(28, Lk)
    dense = rnd(29, Lq, Lk)
    dense[dense < 0.3] = NEG_INF
    dense[2] = NEG_INF                     # one fully masked row
    A = mask_matrix(kind, Lq, Lk, window_left=9, dense=dense, zh_row=zh, keep_k=20)
    o1, l1 = attention_rows_ref(q, k, v, 0.25, A)
    o2, l2 = attention_chunked_ref(q, k, v, 0.25, A, chunk)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    fin = np.isfinite(l1)
    np.testing.assert_array_equal(np.isfinite(l2), fin)
    np.testing.assert_allclose(l2[fin], l1[fin], rtol=0, atol=1e-12)


def test_executorch_window_case_guard():
    """ExecuTorch page, 'Summary': 700-key cache, position 575, window 60, chunk 512."""
    g = json.load(open(os.path.join(GOLDEN, "executorch_window_case.json")))
    Lk, pos, W, chunk = g["Lk"], g["position"], g["window_left"], g["chunk"]
    d = 32
    # a decode step: one query row at absolute position 575 against the 700-key cache
    positions = np.array([pos, 560])
    A = np.stack([np.where((np.arange(Lk) >= p - W) & (np.arange(Lk) <= p), 0.0, NEG_INF) for p in positions])
    vis = np.flatnonzero(np.isfinite(A[0]))
    assert vis[0] == g["first_visible_key"] and vis[-1] == g["last_visible_key"]
    assert vis.size == g["n_visible"]
    assert np.all(A[0, :chunk] == NEG_INF) == g["first_chunk_fully_masked"]
    q, k, v = rnd(30, 2, d), rnd(31, Lk, d), rnd(32, Lk, d)
    o_ref, l_ref = attention_rows_ref(q, k, v, 1 / np.sqrt(d), A)
    for c in (1, 7, 64, 512):
        o, l = attention_chunked_ref(q, k, v, 1 / np.sqrt(d), A, c)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)
        o_bad, _ = attention_chunked_ref(q, k, v, 1 / np.sqrt(d), A, c, guard=False)
        assert np.isnan(o_bad[0]).all()          # row 575: leading all -inf chunk -> NaN
        if c == 512:
            assert not np.isnan(o_bad[1]).any()  # row 560 still sees keys 500..511 in chunk 0


# ---------------------------------------------------------------- causal alignment
def test_bottom_right_causal_equals_padded_queries():
    """FastChat page: past keys without padding q must equal padding q up to kv_len."""
    Lq, Lk, d = 5, 17, 8
    q, k, v = rnd(33, 1, 1, Lq, d), rnd(34, 1, 1, Lk, d), rnd(35, 1, 1, Lk, d)
    out, lse = attention_ref(q, k, v, 0.6, "causal")
    qpad = np.concatenate([rnd(36, 1, 1, Lk - Lq, d) * 100.0, q], axis=2)
    outp, lsep = attention_ref(qpad, k, v, 0.6, "causal")
    np.testing.assert_allclose(out, outp[:, :, Lk - Lq:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lsep[:, :, Lk - Lq:], rtol=0, atol=1e-13)


def test_square_causal_matches_torch_top_left():
    B, H, L, d = 2, 3, 37, 16
    q, k, v = rnd(37, B, H, L, d), rnd(38, B, H, L, d), rnd(39, B, H, L, d)
    out, _ = attention_ref(q, k, v, 0.2, "causal")
    np.testing.assert_allclose(out, torch_sdpa(q, k, v, 0.2, causal=True), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["none", "causal", "window", "dense", "topk"])
def test_matches_torch_sdpa_with_materialised_mask(kind):
    """Library routine pin (fp64 CPU): GQA by torch's enable_gqa, mask as additive float."""
    B, Hq, Hkv, Lq, Lk, d = 2, 4, 2, 11, 45, 16
    q, k, v = rnd(40, B, Hq, Lq, d), rnd(41, B, Hkv, Lk, d), rnd(42, B, Hkv, Lk, d)
    zh = rnd(43, B, Hkv, Lk)
    dense = rnd(44, Lq, Lk)
    dense[dense > 0.8] = NEG_INF
    out, lse = attention_ref(q, k, v, 0.3, kind, window_left=6, mask=dense, zero_hold=zh, keep_k=7)
    G = Hq // Hkv
    A = np.zeros((B, Hq, Lq, Lk))
    for b in range(B):
        for h in range(Hq):
            A[b, h] = mask_matrix(kind, Lq, Lk, window_left=6, dense=dense, zh_row=zh[b, h // G], keep_k=7)
    live = np.isfinite(A).any(axis=-1)
    ref = torch_sdpa(q, k, v, 0.3, A=A)
    np.testing.assert_allclose(out[live], ref[live], rtol=0, atol=1e-12)
    assert np.all(out[~live] == 0) and np.all(lse[~live] == NEG_INF)


# ---------------------------------------------------------------- window / dense / GQA
def test_window_kind_equals_dense_window_mask_two_routes():
    """A dense [16,700] window-60 mask for positions 560..575 equals the window kind over
    the first 576 keys, where bottom-right alignment puts row i at 560+i."""
    from synth import window_dense_mask
    B, Hq, Hkv, d = 1, 4, 1, 16
    q, k, v = rnd(45, B, Hq, 16, d), rnd(46, B, Hkv, 700, d), rnd(47, B, Hkv, 700, d)
    o1, l1 = attention_ref(q, k, v, 0.25, "dense", mask=window_dense_mask(16, 700, 560, 60))
    o2, l2 = attention_ref(q, k[:, :, :576], v[:, :, :576], 0.25, "window", window_left=60)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    B, Hq, Hkv, Lq, Lk, d = 2, 8, 2, 9, 31, 8
    q, k, v = rnd(48, B, Hq, Lq, d), rnd(49, B, Hkv, Lk, d), rnd(50, B, Hkv, Lk, d)
    zh = rnd(51, B, Hkv, Lk)
    for kind in ("causal", "topk"):
        o1, l1 = attention_ref(q, k, v, 0.4, kind, zero_hold=zh, keep_k=5)
        G = Hq // Hkv
        o2, l2 = attention_ref(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.4, kind,
                               zero_hold=np.repeat(zh, G, axis=1), keep_k=5)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


def test_gqa_rejects_indivisible_heads():
    q, k = np.zeros((1, 3, 2, 4)), np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        attention_ref(q, k, k, 1.0, "none")


def test_dense_mask_column_permutation_invariance():
    Lq, Lk, d = 6, 40, 8
    q, k, v = rnd(52, Lq, d), rnd(53, Lk, d), rnd(54, Lk, d)
    A = rnd(55, Lq, Lk)
    A[A < -0.5] = NEG_INF
    perm = np.random.default_rng(56).permutation(Lk)
    o1, l1 = attention_rows_ref(q, k, v, 0.5, A)
    o2, l2 = attention_rows_ref(q, k[perm], v[perm], 0.5, A[:, perm])
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


def test_dense_mask_values_are_added_to_logits_not_weights():
    """A finite mask shifts the logits: for two visible keys the weight ratio is exp(delta)."""
    q = np.zeros((1, 4))
    k = np.zeros((2, 4))
    v = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    A = np.array([[0.0, np.log(3.0)]])
    out, lse = attention_rows_ref(q, k, v, 1.0, A)
    np.testing.assert_allclose(out[0, :2], [0.25, 0.75], rtol=0, atol=1e-15)
    assert abs(lse[0] - np.log(4.0)) < 1e-15


# ---------------------------------------------------------------- top-k
def brute_kept(zh, Lq, keep_k, causal=True):
    """Count, for each allowed key, how many allowed keys beat it (larger value, or equal
    value and lower index); keep it iff fewer than keep_k do."""
    Lk = len(zh)
    pos = query_positions(Lq, Lk)
    kept = np.zeros((Lq, Lk), dtype=bool)
    for i in range(Lq):
        allowed = [j for j in range(Lk) if (j <= pos[i] or not causal)]
        for j in allowed:
            beaters = sum(1 for m in allowed if zh[m] > zh[j] or (zh[m] == zh[j] and m < j))
            kept[i, j] = beaters < keep_k
    return kept


def expiry_kept(zh, Lq, keep_k):
    """Second encoding: key j stays in its prefix's top-k from position j until the first
    position e_j >= j at which keep_k keys beating it have been seen; kept iff j <= p_i < e_j."""
    Lk = len(zh)
    e = np.full(Lk, np.iinfo(np.int64).max)
    for j in range(Lk):
        seen = 0
        for p in range(Lk):
            if zh[p] > zh[j] or (zh[p] == zh[j] and p < j):
                seen += 1
            if p >= j and seen >= keep_k:
                e[j] = p
                break
    pos = query_positions(Lq, Lk)
    return (np.arange(Lk)[None, :] <= pos[:, None]) & (pos[:, None] < e[None, :])


def test_topk_minimal_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "minimal_topk_example.json")))
    for case in g["cases"]:
        zh = np.array([float(x) for x in case["zero_hold"]])
        Lq, keep_k = case["Lq"], case["keep_k"]
        kept = topk_kept_ref(zh, Lq, keep_k)
        want = np.zeros_like(kept)
        for i, ks in enumerate(case["kept"]):
            want[i, ks] = True
        np.testing.assert_array_equal(kept, want, err_msg=case["name"])
        rank = topk_rank_ref(zh)
        np.testing.assert_array_equal(rank, case["rank"], err_msg=case["name"])
        tau = topk_tau_ref(rank, Lq, keep_k)
        np.testing.assert_array_equal(tau, case["tau"], err_msg=case["name"])
        np.testing.assert_array_equal(kept_from_rank_tau(rank, tau, Lq), want)


def test_topk_every_tie_pattern_against_brute_force():
    vals = [-1.0, -0.0, 0.0, 1.0]
    Lk = 4
    for code in range(4 ** Lk):
        zh = np.array([vals[(code >> (2 * t)) & 3] for t in range(Lk)])
        for keep_k in (1, 2, 3, 4):
            for Lq in (4, 2):
                want = brute_kept(zh, Lq, keep_k)
                np.testing.assert_array_equal(topk_kept_ref(zh, Lq, keep_k), want)
                rank = topk_rank_ref(zh)
                tau = topk_tau_ref(rank, Lq, keep_k)
                np.testing.assert_array_equal(kept_from_rank_tau(rank, tau, Lq), want)
            nc = brute_kept(zh, 4, keep_k, causal=False)
            np.testing.assert_array_equal(topk_kept_ref(zh, 4, keep_k, causal=False), nc)


def test_topk_random_against_brute_force_and_expiry():
    rng = np.random.default_rng(57)
    for t in range(120):
        Lk = int(rng.integers(1, 25))
        Lq = int(rng.integers(1, Lk + 3))
        keep_k = int(rng.integers(1, Lk + 2))
        zh = rng.integers(-3, 4, size=Lk).astype(np.float64) * rng.choice([1.0, 0.5])
        zh[rng.random(Lk) < 0.2] = -0.0
        want = brute_kept(zh, Lq, keep_k)
        np.testing.assert_array_equal(topk_kept_ref(zh, Lq, keep_k), want)
        np.testing.assert_array_equal(expiry_kept(zh, Lq, keep_k), want)
        rank = topk_rank_ref(zh)
        np.testing.assert_array_equal(kept_from_rank_tau(rank, topk_tau_ref(rank, Lq, keep_k), Lq), want)


def test_topk_special_cases():
    Lk, d = 30, 8
    zh = rnd(58, Lk)
    # keep_k >= allowed: the causal mask plus the bias
    kept = topk_kept_ref(zh, Lk, Lk)
    np.testing.assert_array_equal(kept, np.tril(np.ones((Lk, Lk), dtype=bool)))
    # keep_k = 1 keeps the prefix argmax (lowest index on ties), so out is that key's V row
    zt = np.round(zh * 2) / 2
    kept1 = topk_kept_ref(zt, Lk, 1)
    for i in range(Lk):
        assert np.flatnonzero(kept1[i]).tolist() == [int(np.argmax(zt[: i + 1]))]
    q, k, v = rnd(59, 1, 1, Lk, d), rnd(60, 1, 1, Lk, d), rnd(61, 1, 1, Lk, d)
    out, _ = attention_ref(q, k, v, 0.5, "topk", zero_hold=zt[None, None], keep_k=1)
    for i in range(Lk):
        np.testing.assert_array_equal(out[0, 0, i], v[0, 0, int(np.argmax(zt[: i + 1]))])
    # all-equal values keep the lowest keep_k indices
    kept_eq = topk_kept_ref(np.zeros(Lk), Lk, 4)
    for i in range(Lk):
        assert np.flatnonzero(kept_eq[i]).tolist() == list(range(min(4, i + 1)))
    # the kept key's zero_hold value is added to its logit
    out_b, lse_b = attention_ref(q, k, v, 0.5, "topk", zero_hold=zt[None, None], keep_k=Lk)
    out_c, lse_c = attention_ref(q, k, v, 0.5, "causal")
    assert not np.allclose(lse_b, lse_c)
    A = np.where(np.tril(np.ones((Lk, Lk))) > 0, zt[None, :], NEG_INF)
    o_d, l_d = attention_ref(q, k, v, 0.5, "dense", mask=A)
    np.testing.assert_allclose(out_b, o_d, rtol=0, atol=1e-14)


def test_topk_tau_is_int32_max_when_all_allowed_kept():
    rank = topk_rank_ref(rnd(62, 10))
    tau = topk_tau_ref(rank, 10, 4)
    assert np.all(tau[:4] == INT32_MAX) and np.all(tau[4:] < 10)


def test_pack_keep_bits_matches_numpy_packbits():
    kept = np.random.default_rng(63).random((3, 5, 70)) < 0.4
    words = pack_keep_bits(kept)
    ref = np.packbits(np.pad(kept, ((0, 0), (0, 0), (0, 26))), axis=-1, bitorder="little")
    np.testing.assert_array_equal(words, ref.view(np.uint32))


# ---------------------------------------------------------------- split-KV merge
def test_lse_merge_of_any_partition_equals_unsplit():
    Lq, Lk, d = 7, 90, 8
    q, k, v = rnd(64, Lq, d), rnd(65, Lk, d), rnd(66, Lk, d)
    A = mask_matrix("window", Lq, Lk, window_left=20)     # leading parts fully masked
    o_ref, l_ref = attention_rows_ref(q, k, v, 0.4, A)
    rng = np.random.default_rng(67)
    for t in range(20):
        cuts = np.sort(rng.choice(np.arange(1, Lk), size=int(rng.integers(1, 8)), replace=False))
        bounds = [0, *cuts.tolist(), Lk]
        outs, lses = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            o, l = attention_rows_ref(q, k[a:b], v[a:b], 0.4, A[:, a:b])
            outs.append(o)
            lses.append(l)
        o_m, l_m = lse_merge_ref(np.stack(outs), np.stack(lses))
        np.testing.assert_allclose(o_m, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_m, l_ref, rtol=0, atol=1e-12)
    o_dead, l_dead = lse_merge_ref(np.zeros((3, 2, d)), np.full((3, 2), NEG_INF))
    assert np.all(o_dead == 0) and np.all(l_dead == NEG_INF)
