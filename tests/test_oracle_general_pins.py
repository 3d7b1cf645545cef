"""Pins for oracle/general.py (score modifiers, per-head dense masks, top-k variants),
checked against facts fixed outside that module: limits and closed forms of softcap, a
library routine (torch's CPU fp64 attention with a mask built from the logistic
function), a second route for ALiBi (its bias folded into an extra key dimension, with
the two sides of the query position merged by log-sum-exp), broadcast against
materialised masks, and the top-k brute force. No GPU is used here."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_ref, attention_rows_ref, lse_merge_ref, mask_matrix, query_positions, topk_kept_ref
from oracle.general import general_attention_ref


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def problem(seed, B=2, Hq=4, Hkv=2, Lq=7, Lk=19, d=8):
    return rnd(seed, B, Hq, Lq, d), rnd(seed + 1, B, Hkv, Lk, d), rnd(seed + 2, B, Hkv, Lk, d)


def head_kv(k, v, Hq):
    G = Hq // k.shape[1]
    return np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)


@pytest.mark.parametrize("kind", ["none", "causal", "window", "dense", "topk"])
def test_without_modifiers_equals_the_base_oracle(kind):
    q, k, v = problem(10)
    B, Hq, Lq, _ = q.shape
    Lk = k.shape[2]
    mask = rnd(13, Lq, Lk) if kind == "dense" else None
    zh = rnd(14, B, 2, Lk) if kind == "topk" else None
    o1, l1 = attention_ref(q, k, v, 0.4, kind, window_left=3, mask=mask, zero_hold=zh, keep_k=5)
    o2, l2 = general_attention_ref(q, k, v, 0.4, kind, window_left=3, mask=mask, zero_hold=zh, keep_k=5)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-14)


# ------------------------------------------------------------------------ softcap
def test_softcap_vanishes_as_the_cap_grows():
    """cap * tanh(t / cap) -> t as cap -> infinity (a cap that multiplied or divided the
    wrong way would not reach the plain result)."""
    q, k, v = problem(20)
    o1, l1 = attention_ref(q, k, v, 0.4, "causal")
    o2, l2 = general_attention_ref(q, k, v, 0.4, "causal", softcap=1e7)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-10)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-10)


def test_tiny_softcap_flattens_the_logits():
    """cap -> 0 squeezes every logit into (-cap, cap): the output tends to the mean of the
    visible V rows and LSE to ln(#visible)."""
    q, k, v = problem(21)
    Lq, Lk = q.shape[2], k.shape[2]
    o, lse = general_attention_ref(q, k, v, 0.4, "causal", softcap=1e-9)
    kk, vv = head_kv(k, v, q.shape[1])
    pos = query_positions(Lq, Lk)
    for i in range(Lq):
        n = pos[i] + 1
        np.testing.assert_allclose(o[:, :, i], vv[:, :, :n].mean(axis=2), rtol=0, atol=1e-8)
        np.testing.assert_allclose(lse[:, :, i], np.log(n), rtol=0, atol=1e-8)


def test_softcap_single_visible_key():
    """One visible key: output = its V row, LSE = the capped logit of that key."""
    q, k, v = problem(22, B=1, Hq=1, Hkv=1, Lq=5, Lk=12)
    cap = 0.7
    o, lse = general_attention_ref(q, k, v, 0.9, "window", window_left=0, softcap=cap)
    pos = query_positions(5, 12)
    np.testing.assert_array_equal(o[0, 0], v[0, 0, pos])
    t = 0.9 * np.einsum("id,id->i", q[0, 0], k[0, 0, pos])
    np.testing.assert_allclose(lse[0, 0], cap * np.tanh(t / cap), rtol=0, atol=1e-15)


def test_softcap_matches_torch_with_a_logistic_mask():
    """tanh(x) = 2*sigmoid(2x) - 1: the capped logits built with torch.sigmoid from the
    scaled scores, turned into an additive mask over torch's own attention (fp64)."""
    q, k, v = problem(23, B=1, Hq=2, Hkv=2, Lq=6, Lk=11, d=16)
    cap, scale = 1.3, 0.8
    o, lse = general_attention_ref(q, k, v, scale, "none", softcap=cap)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    t = scale * (tq @ tk.transpose(-1, -2))
    capped = cap * (2 * torch.sigmoid(2 * t / cap) - 1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=capped - t, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(capped, dim=-1).numpy(), rtol=0, atol=1e-13)


# ------------------------------------------------------------------------ ALiBi
def test_zero_slopes_change_nothing():
    q, k, v = problem(30)
    o1, l1 = attention_ref(q, k, v, 0.4, "window", window_left=4)
    o2, l2 = general_attention_ref(q, k, v, 0.4, "window", window_left=4, alibi_slopes=np.zeros(4))
    np.testing.assert_array_equal(o2, o1)
    np.testing.assert_array_equal(l2, l1)


def folded_side(q_row, k, v, scale, slope, pos, keys, sign):
    """Plain attention of one query row over `keys`, with the ALiBi bias of that side
    folded into one more dimension: for keys j on one side of pos, -slope*|pos - j| =
    sign*slope*j - sign*slope*pos; the first part rides on an extra key feature, the
    constant is added back to the LSE."""
    qe = np.concatenate([q_row, [1.0]])[None, :]
    ke = np.concatenate([k[keys], (sign * slope * keys / scale)[:, None]], axis=1)
    o, l = attention_rows_ref(qe, ke, v[keys], scale, np.zeros((1, keys.size)))
    return o[0], l[0] - sign * slope * pos


@pytest.mark.parametrize("kind", ["causal", "none"])
def test_alibi_equals_bias_folded_into_an_extra_key_dimension(kind):
    """Keys at or before the query position get slope*(j - p), keys after it slope*(p - j):
    each side is plain attention with one extra key feature; the two sides are merged by
    log-sum-exp (lse_merge_ref, pinned on its own)."""
    q, k, v = problem(31, B=1, Hq=4, Hkv=2, Lq=5, Lk=13)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625])
    scale = 0.6
    o, lse = general_attention_ref(q, k, v, scale, kind, alibi_slopes=slopes)
    Lq, Lk = q.shape[2], k.shape[2]
    pos = query_positions(Lq, Lk)
    for h in range(4):
        g = h // 2
        for i in range(Lq):
            p = int(pos[i])
            left = np.arange(0, p + 1)
            oL, lL = folded_side(q[0, h, i], k[0, g], v[0, g], scale, slopes[h], p, left, +1.0)
            if kind == "causal" or p + 1 >= Lk:
                ref_o, ref_l = oL, lL
            else:
                right = np.arange(p + 1, Lk)
                oR, lR = folded_side(q[0, h, i], k[0, g], v[0, g], scale, slopes[h], p, right, -1.0)
                ref_o, ref_l = lse_merge_ref(np.stack([oL, oR]), np.array([lL, lR]))
            np.testing.assert_allclose(o[0, h, i], ref_o, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[0, h, i], ref_l, rtol=0, atol=1e-13)


def test_alibi_uses_the_bottom_right_position():
    """With past keys, the distance is from the row's absolute position: the last query
    row of a block against the newest key has distance 0, so a huge slope keeps only the
    newest key (output = its V row) and the key just before the row is attended."""
    q, k, v = problem(32, B=1, Hq=1, Hkv=1, Lq=3, Lk=9)
    o, _ = general_attention_ref(q, k, v, 0.5, "causal", alibi_slopes=np.array([200.0]))
    pos = query_positions(3, 9)
    np.testing.assert_allclose(o[0, 0], v[0, 0, pos], rtol=0, atol=1e-12)


# ------------------------------------------------------------------------ per-head dense masks
def test_broadcast_mask_equals_the_single_mask():
    q, k, v = problem(40)
    Lq, Lk = q.shape[2], k.shape[2]
    m = rnd(43, Lq, Lk)
    m[m < -1.0] = -np.inf
    o1, l1 = attention_ref(q, k, v, 0.4, "dense", mask=m)
    o2, l2 = general_attention_ref(q, k, v, 0.4, "dense", mask=m[None, None])
    np.testing.assert_array_equal(o2, o1)
    np.testing.assert_array_equal(l2, l1)


@pytest.mark.parametrize("shape", [(2, 4), (1, 4), (2, 1)])
def test_per_head_mask_equals_each_slice_run_alone(shape):
    """A mask with its own slice per (b, h) (or per b, or per h): each head equals the
    single-mask oracle run with that head's slice."""
    q, k, v = problem(41)
    B, Hq, Lq, _ = q.shape
    Lk = k.shape[2]
    m = rnd(44, *shape, Lq, Lk)
    m[m < -1.2] = -np.inf
    o, lse = general_attention_ref(q, k, v, 0.4, "dense", mask=m)
    for b in range(B):
        for h in range(Hq):
            sl = m[b if shape[0] > 1 else 0, h if shape[1] > 1 else 0]
            o1, l1 = attention_ref(q[b:b + 1, h:h + 1], k[b:b + 1, h // 2:h // 2 + 1], v[b:b + 1, h // 2:h // 2 + 1],
                                   0.4, "dense", mask=sl)
            np.testing.assert_array_equal(o[b, h], o1[0, 0])
            np.testing.assert_array_equal(lse[b, h], l1[0, 0])


# ------------------------------------------------------------------------ top-k variants
def brute_kept_all(zh, keep_k):
    """Global top-k by counting: key j is kept iff fewer than keep_k keys come before it in
    the order (larger value, or equal value and lower index); -0.0 equals +0.0."""
    z = np.where(zh == 0.0, 0.0, zh)
    before = (z[None, :] > z[:, None]) | ((z[None, :] == z[:, None]) & (np.arange(z.size)[None, :] < np.arange(z.size)[:, None]))
    return before.sum(axis=1) < keep_k


def test_noncausal_topk_attention_against_brute_force_keep_set():
    q, k, v = problem(50, B=1, Hq=2, Hkv=2, Lq=6, Lk=10)
    zh = np.round(rnd(51, 1, 2, 10), 0)  # ties
    zh[0, 0, 3] = -0.0
    o, lse = general_attention_ref(q, k, v, 0.5, "topk", zero_hold=zh, keep_k=4, topk_causal=False)
    for h in range(2):
        keep = brute_kept_all(zh[0, h], 4)
        A = np.where(keep[None, :], zh[0, h][None, :], -np.inf).repeat(6, axis=0)
        o1, l1 = attention_rows_ref(q[0, h], k[0, h], v[0, h], 0.5, A)
        np.testing.assert_allclose(o[0, h], o1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, h], l1, rtol=0, atol=1e-14)
    # every row keeps the same set, including rows whose position precedes kept keys
    np.testing.assert_array_equal(topk_kept_ref(zh[0, 0], 6, 4, causal=False),
                                  np.tile(brute_kept_all(zh[0, 0], 4), (6, 1)))


@pytest.mark.parametrize("causal", [True, False])
def test_topk_with_dense_mask_adds_both_to_kept_keys(causal):
    """Kept keys get zero_hold + mask; the rest -inf: equal to the dense kind with that
    combined mask (the dense kind is pinned against torch)."""
    q, k, v = problem(52, B=1, Hq=2, Hkv=1, Lq=5, Lk=12)
    zh = rnd(53, 1, 1, 12)
    m = rnd(54, 5, 12)
    m[1, 3] = -np.inf
    o, lse = general_attention_ref(q, k, v, 0.5, "topk", zero_hold=zh, keep_k=3, topk_causal=causal, mask=m)
    kept = topk_kept_ref(zh[0, 0], 5, 3, causal=causal)
    combined = np.where(kept, zh[0, 0][None, :] + m, -np.inf)
    o1, l1 = attention_ref(q, k, v, 0.5, "dense", mask=combined)
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, l1, rtol=0, atol=1e-14)


def test_modifiers_compose_in_order():
    """softcap applies to the scaled scores only: ALiBi and the mask are added after it, so
    a huge cap with ALiBi equals ALiBi alone, and a mask shift moves only the LSE."""
    q, k, v = problem(60)
    slopes = np.array([0.3, 0.2, 0.1, 0.05])
    o1, l1 = general_attention_ref(q, k, v, 0.4, "causal", alibi_slopes=slopes)
    o2, l2 = general_attention_ref(q, k, v, 0.4, "causal", alibi_slopes=slopes, softcap=1e7)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-10)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-10)
    Lq, Lk = q.shape[2], k.shape[2]
    m = mask_matrix("causal", Lq, Lk)
    o3, l3 = general_attention_ref(q, k, v, 0.4, "dense", mask=m + 2.5, alibi_slopes=slopes, softcap=0.9)
    o4, l4 = general_attention_ref(q, k, v, 0.4, "dense", mask=m, alibi_slopes=slopes, softcap=0.9)
    np.testing.assert_allclose(o3, o4, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l3, l4 + 2.5, rtol=0, atol=1e-13)


def one_key_mask(Lq, Lk, keys):
    """Dense mask that leaves key keys[i] visible to row i and hides every other key."""
    m = np.full((Lq, Lk), -np.inf)
    m[np.arange(Lq), keys] = 0.0
    return m


def test_softcap_then_alibi_single_key_closed_form():
    """One visible key at distance delta from the row: LSE = cap*tanh(t/cap) - slope*delta
    and the output is that key's V row. Applying ALiBi inside the tanh (the other order)
    gives cap*tanh((t - slope*delta)/cap) instead, which differs here by more than 0.1."""
    q, k, v = problem(61, B=1, Hq=2, Hkv=1, Lq=4, Lk=10)
    Lq, Lk = 4, 10
    pos = query_positions(Lq, Lk)
    keys = np.array([0, 2, 9, 5])  # distances 6, 5, 2 (a key after the row) and 4
    cap, scale = 0.8, 0.9
    slopes = np.array([0.35, 0.6])
    o, lse = general_attention_ref(q, k, v, scale, "dense", mask=one_key_mask(Lq, Lk, keys), alibi_slopes=slopes,
                                   softcap=cap)
    for h in range(2):
        t = scale * np.einsum("id,id->i", q[0, h], k[0, 0, keys])
        delta = np.abs(pos - keys)
        np.testing.assert_array_equal(o[0, h], v[0, 0, keys])
        np.testing.assert_allclose(lse[0, h], cap * np.tanh(t / cap) - slopes[h] * delta, rtol=0, atol=1e-15)
        swapped = cap * np.tanh((t - slopes[h] * delta) / cap)
        assert np.abs(swapped - lse[0, h]).min() > 0.1


def test_softcap_then_alibi_two_keys_weights():
    """Two visible keys a and b: the output is w*v_a + (1-w)*v_b with
    w = 1 / (1 + exp(z_b - z_a)), z = cap*tanh(t/cap) - slope*|p - j|, and
    LSE = z_a + log(1 + exp(z_b - z_a))."""
    q, k, v = problem(62, B=1, Hq=1, Hkv=1, Lq=1, Lk=8)
    p = 7
    a, b = 1, 6
    m = np.full((1, 8), -np.inf)
    m[0, [a, b]] = 0.0
    cap, scale, slope = 0.5, 1.1, 0.4
    o, lse = general_attention_ref(q, k, v, scale, "dense", mask=m, alibi_slopes=np.array([slope]), softcap=cap)
    za = cap * np.tanh(scale * q[0, 0, 0] @ k[0, 0, a] / cap) - slope * (p - a)
    zb = cap * np.tanh(scale * q[0, 0, 0] @ k[0, 0, b] / cap) - slope * (p - b)
    w = 1.0 / (1.0 + np.exp(zb - za))
    np.testing.assert_allclose(o[0, 0, 0], w * v[0, 0, a] + (1 - w) * v[0, 0, b], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 0], za + np.log1p(np.exp(zb - za)), rtol=0, atol=1e-14)


def test_softcap_and_alibi_match_torch_with_both_in_the_mask():
    """Library route with both modifiers: torch's fp64 attention over the scaled scores with
    an additive mask that replaces each score by its capped value (built from
    torch.sigmoid) and subtracts the ALiBi distance term, under the causal mask."""
    q, k, v = problem(63, B=1, Hq=2, Hkv=2, Lq=5, Lk=9, d=16)
    cap, scale = 1.1, 0.7
    slopes = np.array([0.45, 0.15])
    o, lse = general_attention_ref(q, k, v, scale, "causal", alibi_slopes=slopes, softcap=cap)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    t = scale * (tq @ tk.transpose(-1, -2))
    capped = cap * (2 * torch.sigmoid(2 * t / cap) - 1)
    pos = torch.from_numpy(query_positions(5, 9)).double()[:, None]
    j = torch.arange(9, dtype=torch.float64)[None, :]
    bias = -torch.from_numpy(slopes)[:, None, None] * (pos - j).abs()[None]
    causal = torch.where(j <= pos, 0.0, -torch.inf)[None]
    z = capped + bias[None] + causal[None]
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=z - t, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-13)
