"""Randomised shapes on the GPU against the fp64 oracle: forward (attn_fwd) and backward
(attn_bwd) over seeded draws of batch, head counts and grouping, lengths (Lq above, equal to
and below Lk, one-row and one-key cases), head dim, dtype and mask kind with its parameters;
varlen batches (attn_fwd_varlen) over seeded draws of sequence count and lengths (empty
queries, no keys, fewer keys than queries), page size, the cache/new-token split, ALiBi,
softcap and forced KV splits; attn_fwd_ex over seeded draws of memory layouts (transposed
cache, padded rows), dense masks broadcast over batch and head, top-k over causal or all
keys, ALiBi and softcap on every mask kind, and forced paths and splits; dynamic_mask_topk
over seeded draws of lengths on both sides of the merge/count switch, keep counts and tie-heavy
zero_hold values (bit-exact). Every draw is printed before it runs, so a failure names its
case."""
import numpy as np
import pytest

import synth
from helpers import compare, run_gpu, run_oracle, say

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


KINDS = ["none", "causal", "window", "dense", "topk"]


def draw_case(i, dtypes):
    rng = np.random.default_rng(5000 + i)
    dtype = dtypes[rng.integers(len(dtypes))]
    d = int(rng.choice([64, 128])) if dtype != "fp32" else int(rng.choice([8, 40, 64, 96, 128, 256]))
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    Lk = int(rng.choice([1, 2, 31, 64, 65, 127, 200, 513, 700]))
    Lq = int(rng.choice([1, 2, 7, 32, 33, 100, 256])) if rng.random() < 0.8 else Lk
    kind = KINDS[rng.integers(len(KINDS))]
    wl = int(rng.integers(0, 80))
    keep = int(rng.integers(1, max(2, Lk + 1)))
    mask = None
    if kind == "dense":
        mask = rng.standard_normal((Lq, Lk)).astype(np.float32)
        mask[rng.random((Lq, Lk)) < rng.uniform(0.0, 0.9)] = -np.inf
    return dict(dtype=dtype, d=d, B=B, Hq=Hkv * G, Hkv=Hkv, Lq=Lq, Lk=Lk, kind=kind, window_left=wl, keep_k=keep,
                mask=mask, seed=6000 + i)


def problem(c, label):
    return synth.make_problem(
        f"{label} {c['dtype']} d{c['d']} B{c['B']} H{c['Hq']}/{c['Hkv']} {c['Lq']}x{c['Lk']} {c['kind']} "
        f"wl{c['window_left']} keep{c['keep_k']}", c["B"], c["Hq"], c["Hkv"], c["Lq"], c["Lk"], c["d"], c["dtype"],
        c["kind"], c["seed"], window_left=c["window_left"], keep_k=c["keep_k"], with_zero_hold=c["kind"] == "topk",
        mask=c["mask"])


@pytest.mark.parametrize("i", range(60))
def test_forward_random(i):
    p = problem(draw_case(i, ["bf16", "fp16", "fp32"]), f"random fwd #{i}")
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


@pytest.mark.parametrize("i", range(30))
def test_backward_random(i):
    from test_gpu_bwd import check
    c = draw_case(100 + i, ["bf16", "fp16"])
    if c["Hq"] // c["Hkv"] > 128:
        pytest.skip("more than 128 query heads per KV head")
    check(problem(c, f"random bwd #{i}"), 7000 + i)


def draw_varlen(i):
    rng = np.random.default_rng(9000 + i)
    S = int(rng.integers(1, 9))
    q_lens = [int(rng.choice([0, 1, 1, 2, 5, 37, 64, 65, 130, 257])) for _ in range(S)]
    if max(q_lens) == 0:
        q_lens[0] = 1
    k_lens = [int(rng.choice([0, 1, 3])) if rng.random() < 0.15 else q + int(rng.integers(0, 700)) for q in q_lens]
    Hkv = int(rng.integers(1, 4))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8, 16]))
    dtype = ["bf16", "fp16"][rng.integers(2)]
    d = int(rng.choice([64, 128]))
    kind = ["none", "causal", "window"][rng.integers(3)]
    wl = int(rng.integers(0, 150))
    page = int(rng.choice([0, 1, 8, 16, 32, 128]))
    two = bool(rng.random() < 0.3)
    alibi = [float(2.0 ** -rng.uniform(0.5, 8.0)) for _ in range(Hq)] if rng.random() < 0.3 else None
    softcap = float(rng.uniform(5.0, 50.0)) if rng.random() < 0.3 else 0.0
    splits = int(rng.integers(2, 8)) if rng.random() < 0.2 else 0
    name = (f"random varlen #{i} {dtype} d{d} H{Hq}/{Hkv} q{q_lens} k{k_lens} {kind} wl{wl} page{page} "
            f"two{int(two)} alibi{int(alibi is not None)} softcap{softcap:.1f} splits{splits}")
    p = synth.make_paged_problem(name, q_lens, k_lens, Hq, Hkv, d, dtype, kind, 9500 + i, page_size=page,
                                 two_source=two, window_left=wl)
    return p, alibi, softcap, splits


@pytest.mark.parametrize("i", range(40))
def test_varlen_random(i):
    import masked_flashattention_forward_amd as mfa
    from test_gpu_varlen import check
    p, alibi, softcap, splits = draw_varlen(i)
    mfa.set_debug(force_splits=splits)
    try:
        check(p, alibi=alibi, softcap=softcap)
    finally:
        mfa.set_debug()


def alibi_row_tol(p, kw):
    """Per-row fp32 tolerance of an ALiBi draw. fp32 holds each logit
    z_ij = t_ij - slope_h * |p_i - j| (plus the mask) to a relative 2^-24 = u32, and the
    kernel rounds it a few times on the way (slope times log2 e, the product with the
    distance, the sum with the score, the difference with the running maximum): 4 u32 |z_ij|
    in all. The LSE moves by at most sum_j w_ij |dz_ij| (w the softmax weights), and its own
    final rounding adds u32 |LSE_i|; the output moves by at most twice sum_j w_ij |dz_ij| times
    max|v|. So a row's allowance grows with E_i = sum_j w_ij |z_ij|, the weighted size of its
    logits, not with the far keys it barely sees. Rows whose weight sits on nearby keys keep
    the plain 1e-5."""
    from oracle.attention import query_positions
    from oracle.general import general_mask, general_scores
    G = p.Hq // p.Hkv
    pos = query_positions(p.Lq, p.Lk)
    mask = kw.get("mask")
    full = None if mask is None else np.broadcast_to(mask.astype(np.float64), (p.B, p.Hq, p.Lq, p.Lk))
    q, k = p.f64("q"), p.f64("k")
    cap = float(np.float32(kw.get("softcap", 0.0)))
    E = np.zeros((p.B, p.Hq, p.Lq))
    L = np.zeros((p.B, p.Hq, p.Lq))
    for b in range(p.B):
        for h in range(p.Hq):
            A = general_mask(p.mask_kind, p.Lq, p.Lk, window_left=p.window_left,
                             dense2d=None if full is None else full[b, h],
                             zh_row=None if p.zero_hold is None else p.zero_hold[b, h // G].astype(np.float64),
                             keep_k=p.keep_k, topk_causal=kw["topk_causal"])
            t = general_scores(q[b, h], k[b, h // G], p.scale64, pos, softcap=cap,
                               alibi_slope=float(np.float32(kw["alibi"][h])))
            z = t + A
            vis = np.isfinite(z)
            zm = np.where(vis, z, -np.inf).max(axis=1, keepdims=True)
            zm = np.where(np.isfinite(zm), zm, 0.0)
            w = np.where(vis, np.exp(np.where(vis, z, 0.0) - zm), 0.0)
            tot = w.sum(axis=1, keepdims=True)
            w = w / np.where(tot > 0, tot, 1.0)
            E[b, h] = (w * np.abs(np.where(vis, z, 0.0))).sum(axis=1)
            L[b, h] = np.abs(zm[:, 0] + np.log(np.where(tot[:, 0] > 0, tot[:, 0], 1.0)))
    u = 2.0 ** -24
    return 1e-5 + 8 * u * E * float(np.abs(p.v).max()), 1e-5 + 4 * u * E + u * L


def draw_ex(i):
    from test_gpu_ex import per_head_mask
    rng = np.random.default_rng(11000 + i)
    c = draw_case(300 + i, ["bf16", "fp16", "fp32"])
    c["Hq"] = c["Hkv"] * int(rng.choice([1, 2, 4, 8]))
    c["B"] = int(rng.integers(1, 3))
    if c["kind"] == "dense":
        shape = [(), (c["B"], 1), (1, c["Hq"]), (c["B"], c["Hq"])][rng.integers(4)]
        c["mask"] = per_head_mask(12000 + i, shape, c["Lq"], c["Lk"])
    lays = ["bhld", "blhd", "pad"]
    kw = dict(qlay=lays[rng.integers(3)], klay=lays[rng.integers(3)], olay=lays[rng.integers(3)],
              mask=c["mask"], topk_causal=bool(rng.random() < 0.5))
    if rng.random() < 0.35:
        kw["alibi"] = [float(2.0 ** -rng.uniform(0.5, 8.0)) for _ in range(c["Hq"])]
    if rng.random() < 0.35:
        kw["softcap"] = float(rng.uniform(5.0, 50.0))
    G = c["Hq"] // c["Hkv"]
    r = rng.random()
    if c["dtype"] != "fp32" and r < 0.2:
        kw["path"] = 1
    elif c["dtype"] != "fp32" and r < 0.35 and G * c["Lq"] <= 32:
        kw["path"] = 2
    elif r < 0.45:
        kw["path"] = 0
    if kw.get("path") in (1, 2) and rng.random() < 0.5:
        kw["splits"] = int(rng.integers(2, 8))
    p = problem(c, f"random ex #{i}")
    if c["dtype"] == "fp32" and "alibi" in kw:
        kw["tol"] = alibi_row_tol(p, kw)
    label = (f"{p.name} lay {kw['qlay']}/{kw['klay']}/{kw['olay']} topk_causal{int(kw['topk_causal'])} "
             f"alibi{int('alibi' in kw)} softcap{kw.get('softcap', 0.0):.1f} path{kw.get('path')} "
             f"splits{kw.get('splits', 0)}")
    return p, label, kw


@pytest.mark.parametrize("i", range(40))
def test_ex_random(i):
    from test_gpu_ex import check
    p, label, kw = draw_ex(i)
    check(p, label, **kw)


def draw_topk(i):
    rng = np.random.default_rng(13000 + i)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Lk = int(np.exp(rng.uniform(0.0, np.log(33000.0))))
    Lq = int(rng.integers(1, min(2 * Lk, 40_000_000 // Lk) + 1))
    keep = int(rng.integers(1, Lk + 6))
    causal = bool(rng.random() < 0.5)
    style = int(rng.integers(3))
    if style == 0:    # few distinct values: long tie runs, -0.0 beside +0.0
        zh = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0], dtype=np.float32), size=(B, H, Lk))
    elif style == 1:  # continuous values
        zh = rng.standard_normal((B, H, Lk)).astype(np.float32)
    else:             # continuous with a share of repeated values
        zh = rng.standard_normal((B, H, Lk)).astype(np.float32)
        zh[rng.random(zh.shape) < 0.3] = np.float32(0.25)
    return zh, Lq, keep, causal, f"random topk #{i} B{B} H{H} Lq{Lq} Lk{Lk} keep{keep} causal{int(causal)} style{style}"


@pytest.mark.parametrize("i", range(30))
def test_topk_random(i):
    from test_gpu_topk import check_topk
    zh, Lq, keep, causal, label = draw_topk(i)
    check_topk(zh, Lq, keep, causal, label)
