"""Pins for the varlen / paged-cache oracle (``oracle.paged``), checked against a library
routine (torch's CPU attention in fp64), brute-force scalar loops over explicit page
lookups, and invariants of the cache layout. No GPU is used here."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import paged_attention_ref


def f64(p, name):
    return p.f64(name)


def run_oracle(p):
    return paged_attention_ref(f64(p, "q"), f64(p, "k"), f64(p, "v"), p.cu_seqlens_q, p.cu_seqlens_k,
                               p.block_table, p.page_size, p.scale, p.mask_kind, window_left=p.window_left,
                               k_new=f64(p, "k_new"), v_new=f64(p, "v_new"))


def brute(q, k, v, cu_q, cu_k, table, ps, scale, kind, W=0, k_new=None, v_new=None):
    """Scalar loops: every key fetched by an explicit page lookup, softmax with math.exp."""
    total_q, Hq, d = q.shape
    Hkv = k.shape[-2]
    G = Hq // Hkv
    out = np.zeros((total_q, Hq, d))
    lse = np.full((total_q, Hq), -math.inf)
    for s in range(len(cu_q) - 1):
        Lq, Lk = int(cu_q[s + 1] - cu_q[s]), int(cu_k[s + 1] - cu_k[s])
        ctx = Lk - Lq if k_new is not None else Lk

        def key(j, g, src_cache, src_new):
            if j >= ctx:
                return src_new[int(cu_q[s]) + j - ctx, g]
            if table is None:
                return src_cache[int(cu_k[s]) + j, g]
            return src_cache[int(table[s][j // ps]), j % ps, g]

        if ctx < 0:
            continue
        for i in range(Lq):
            t = int(cu_q[s]) + i
            pos = Lk - Lq + i
            for h in range(Hq):
                g = h // G
                vis = [j for j in range(Lk)
                       if kind == "none" or (j <= pos and (kind == "causal" or j >= pos - W))]
                if not vis:
                    continue
                logits = [scale * sum(q[t, h, c] * key(j, g, k, k_new)[c] for c in range(d)) for j in vis]
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                tot = sum(w)
                for jj, j in enumerate(vis):
                    out[t, h] += (w[jj] / tot) * key(j, g, v, v_new)
                lse[t, h] = m + math.log(tot)
    return out, lse


@pytest.mark.parametrize("kind", ["none", "causal", "window"])
@pytest.mark.parametrize("form", ["paged", "packed", "two_source", "two_source_packed"])
def test_paged_oracle_matches_brute_force(kind, form):
    q_lens = [1, 4, 0, 3, 2, 2]
    k_lens = [7, 9, 5, 3, 0, 1]   # more queries than keys in the last two sequences
    two = form.startswith("two_source")
    if two:                     # every sequence needs Lk >= Lq, except the last (checked dead)
        k_lens = [7, 9, 5, 3, 2, 1]
    p = synth.make_paged_problem("pin", q_lens, k_lens, 4, 2, 5, "fp32", kind, 7,
                                 page_size=0 if form.endswith("packed") else 2, two_source=two,
                                 window_left=2, scale=0.4)
    out, lse = run_oracle(p)
    ob, lb = brute(f64(p, "q"), f64(p, "k"), f64(p, "v"), p.cu_seqlens_q, p.cu_seqlens_k, p.block_table,
                   p.page_size, p.scale, kind, W=2, k_new=f64(p, "k_new"), v_new=f64(p, "v_new"))
    np.testing.assert_allclose(out, ob, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)
    if two:   # the sequence with fewer keys than queries is returned fully masked
        t0 = int(p.cu_seqlens_q[-2])
        assert np.all(out[t0:] == 0) and np.all(np.isneginf(lse[t0:]))


@pytest.mark.parametrize("kind", ["none", "causal"])
def test_equal_lengths_with_identity_pages_match_torch_sdpa(kind):
    """B sequences of L queries over their own L keys, pages in order: the batched dense
    attention of a library routine (square, so torch's top-left causal is bottom-right)."""
    B, L, Hq, Hkv, d, ps = 3, 24, 6, 2, 8, 8
    p = synth.make_paged_problem("pin", [L] * B, [L] * B, Hq, Hkv, d, "fp32", kind, 11, page_size=ps,
                                 spare_pages=0, scale=0.3)
    q, k, v = f64(p, "q"), f64(p, "k"), f64(p, "v")
    pages = L // ps
    ident = np.arange(B * pages, dtype=np.int32).reshape(B, pages)
    qd = q.reshape(B, L, Hq, d).transpose(0, 2, 1, 3)
    kd = k.reshape(B, L, Hkv, d).transpose(0, 2, 1, 3)
    vd = v.reshape(B, L, Hkv, d).transpose(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(np.ascontiguousarray(x)) for x in (qd, kd, vd)),
                                         is_causal=kind == "causal", scale=p.scale, enable_gqa=True).numpy()
    out, lse = paged_attention_ref(q, k, v, p.cu_seqlens_q, p.cu_seqlens_k, ident, ps, p.scale, kind)
    np.testing.assert_allclose(out, ref.transpose(0, 2, 1, 3).reshape(B * L, Hq, d), rtol=0, atol=1e-13)
    # LSE: log of the softmax denominator, from torch's logsumexp of the masked logits
    s = torch.from_numpy(np.einsum("bhid,bhjd->bhij", qd, np.repeat(kd, Hq // Hkv, axis=1)) * p.scale)
    if kind == "causal":
        s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy().transpose(0, 2, 1).reshape(B * L, Hq),
                               rtol=0, atol=1e-12)


def test_page_permutation_does_not_change_the_result():
    p = synth.make_paged_problem("pin", [3, 1, 6], [40, 17, 25], 4, 1, 6, "fp32", "causal", 12, page_size=4)
    out, lse = run_oracle(p)
    perm = np.random.default_rng(5).permutation(p.k.shape[0])
    inv = np.argsort(perm)             # new page perm[i] holds old page i -> new id of old page o is inv[o]
    k2, v2 = f64(p, "k")[perm], f64(p, "v")[perm]
    t2 = inv[p.block_table].astype(np.int32)
    out2, lse2 = paged_attention_ref(f64(p, "q"), k2, v2, p.cu_seqlens_q, p.cu_seqlens_k, t2, p.page_size,
                                     p.scale, "causal")
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_two_source_equals_writing_new_keys_into_the_cache():
    """The cached + active form (vLLM pull request #11277 page, Neuron reply) gives what
    the single-source call gives after the new keys are written to their cache slots."""
    q_lens, k_lens, ps = [2, 5, 1], [9, 5, 13], 4
    p = synth.make_paged_problem("pin", q_lens, k_lens, 4, 2, 6, "fp32", "causal", 13, page_size=ps,
                                 two_source=True)
    out2, lse2 = run_oracle(p)
    # single-source cache: each sequence's pages extended to hold all Lk keys
    S, Hkv, d = len(q_lens), 2, 6
    need = [(lk + ps - 1) // ps for lk in k_lens]
    k1 = np.zeros((sum(need), ps, Hkv, d))
    v1 = np.zeros_like(k1)
    table = np.zeros((S, max(need)), dtype=np.int32)
    nxt = 0
    kc, vc, kn, vn = f64(p, "k"), f64(p, "v"), f64(p, "k_new"), f64(p, "v_new")
    for s in range(S):
        table[s, :need[s]] = np.arange(nxt, nxt + need[s])[::-1]   # pages in reverse order
        nxt += need[s]
        ctx = k_lens[s] - q_lens[s]
        for j in range(k_lens[s]):
            pg, sl = table[s, j // ps], j % ps
            if j < ctx:
                src_pg, src_sl = p.block_table[s, j // ps], j % ps
                k1[pg, sl], v1[pg, sl] = kc[src_pg, src_sl], vc[src_pg, src_sl]
            else:
                r = p.cu_seqlens_q[s] + j - ctx
                k1[pg, sl], v1[pg, sl] = kn[r], vn[r]
    out1, lse1 = paged_attention_ref(f64(p, "q"), k1, v1, p.cu_seqlens_q, p.cu_seqlens_k, table, ps, p.scale,
                                     "causal")
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_packed_equals_paged_with_one_key_per_page():
    p = synth.make_paged_problem("pin", [2, 3, 1], [6, 3, 11], 2, 1, 4, "fp32", "window", 14, page_size=0,
                                 window_left=3)
    out, lse = run_oracle(p)
    k, v = f64(p, "k"), f64(p, "v")
    S = 3
    table = np.zeros((S, max(p.k_lens)), dtype=np.int32)
    for s in range(S):
        table[s, :p.k_lens[s]] = np.arange(p.cu_seqlens_k[s], p.cu_seqlens_k[s + 1])
    out1, lse1 = paged_attention_ref(f64(p, "q"), k[:, None], v[:, None], p.cu_seqlens_q, p.cu_seqlens_k,
                                     table, 1, p.scale, "window", window_left=3)
    np.testing.assert_array_equal(out, out1)
    np.testing.assert_array_equal(lse, lse1)


def test_sequences_are_independent():
    p = synth.make_paged_problem("pin", [2, 4, 3], [8, 4, 12], 4, 2, 4, "fp32", "causal", 15, page_size=4,
                                 spare_pages=0)
    out, lse = run_oracle(p)
    q, k, v = f64(p, "q"), f64(p, "k").copy(), f64(p, "v").copy()
    q = q.copy()
    # perturb everything that belongs to sequence 1: its queries and its pages
    q[p.cu_seqlens_q[1]:p.cu_seqlens_q[2]] += 1.0
    for pg in p.block_table[1, :1]:
        k[pg] += 1.0
        v[pg] -= 1.0
    out2, lse2 = paged_attention_ref(q, k, v, p.cu_seqlens_q, p.cu_seqlens_k, p.block_table, 4, p.scale, "causal")
    a, b = p.cu_seqlens_q[1], p.cu_seqlens_q[2]
    np.testing.assert_array_equal(out2[:a], out[:a])
    np.testing.assert_array_equal(out2[b:], out[b:])
    assert np.abs(out2[a:b] - out[a:b]).max() > 1e-3


def test_sequences_without_queries_or_keys():
    p = synth.make_paged_problem("pin", [0, 3, 2], [5, 0, 4], 2, 2, 4, "fp32", "none", 16, page_size=2)
    out, lse = run_oracle(p)
    assert out.shape == (5, 2, 4)
    np.testing.assert_array_equal(out[:3], 0)          # sequence 1 has no keys
    assert np.all(np.isneginf(lse[:3]))
    assert np.all(np.isfinite(lse[3:]))


def test_alibi_on_causal_sequences_is_a_key_bias_per_head():
    """Causal ALiBi: -slope * (p_i - j) = slope * j - slope * p_i. The row constant leaves
    the softmax unchanged and shifts the LSE by -slope * p_i; slope * j is a key bias, which
    an extra query coordinate 1 against a key coordinate slope * j / scale adds to the
    plain (pinned) paged attention. Positions are each sequence's own, so a sequence-level
    mistake (global key index, shared position) fails here."""
    q_lens, k_lens = [2, 5, 1, 3], [9, 5, 14, 3]
    Hq, Hkv, d = 4, 2, 6
    p = synth.make_paged_problem("pin", q_lens, k_lens, Hq, Hkv, d, "fp32", "causal", 31, page_size=4, scale=0.35)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625])
    out, lse = paged_attention_ref(f64(p, "q"), f64(p, "k"), f64(p, "v"), p.cu_seqlens_q, p.cu_seqlens_k,
                                   p.block_table, p.page_size, p.scale, "causal", alibi_slopes=slopes)
    G = Hq // Hkv
    for h in range(Hq):
        # one head at a time: its slope goes into the key coordinate of its KV head
        q1 = np.concatenate([f64(p, "q")[:, h:h + 1], np.ones((p.total_q, 1, 1))], axis=2)
        kx = np.zeros(p.k.shape[:3] + (1,))
        for s in range(p.num_seqs):
            for j in range(int(k_lens[s])):
                kx[p.block_table[s][j // p.page_size], j % p.page_size, :, 0] = slopes[h] * j / p.scale
        k1 = np.concatenate([f64(p, "k")[:, :, h // G:h // G + 1], kx[:, :, h // G:h // G + 1]], axis=3)
        v1 = np.concatenate([f64(p, "v")[:, :, h // G:h // G + 1], np.zeros(kx.shape[:3] + (1,))[:, :, :1]], axis=3)
        o1, l1 = paged_attention_ref(q1, k1, v1, p.cu_seqlens_q, p.cu_seqlens_k, p.block_table, p.page_size,
                                     p.scale, "causal")
        np.testing.assert_allclose(out[:, h], o1[:, 0, :d], rtol=0, atol=1e-12)
        pos = np.concatenate([np.arange(lq) + lk - lq for lq, lk in zip(q_lens, k_lens)])
        np.testing.assert_allclose(lse[:, h], l1[:, 0] - slopes[h] * pos, rtol=0, atol=1e-11)


def test_softcap_limits_on_paged_sequences():
    """softcap -> infinity is no softcap; a tiny cap flattens every score to ~0 (uniform
    weights over the visible keys: the mean of their values)."""
    p = synth.make_paged_problem("pin", [3, 2], [7, 4], 2, 1, 5, "fp32", "causal", 33, page_size=2, scale=0.4)
    args = (f64(p, "q"), f64(p, "k"), f64(p, "v"), p.cu_seqlens_q, p.cu_seqlens_k, p.block_table, p.page_size,
            p.scale, "causal")
    o0, l0 = paged_attention_ref(*args)
    o1, l1 = paged_attention_ref(*args, softcap=1e9)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)
    o2, l2 = paged_attention_ref(*args, softcap=1e-9)
    vv = f64(p, "v")
    for s, (lq, lk) in enumerate(zip([3, 2], [7, 4])):
        for i in range(lq):
            n = lk - lq + i + 1
            keys = [vv[p.block_table[s][j // 2], j % 2, 0] for j in range(n)]
            t = int(p.cu_seqlens_q[s]) + i
            np.testing.assert_allclose(o2[t, 0], np.mean(keys, axis=0), rtol=0, atol=1e-7)
            np.testing.assert_allclose(l2[t, 0], math.log(n), rtol=0, atol=1e-7)
