"""GPU parity of the varlen / paged forward (attn_fwd_varlen) against the fp64 oracle:
paged, packed and two-source (cached + active) K/V, GQA, decode steps next to prefill
chunks, empty and ragged sequences, split key ranges, and the full serving batch on
sampled sequences."""
import numpy as np
import pytest

import synth
from helpers import compare, run_gpu_paged, run_oracle_paged, say

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


def check(p, alibi=None, softcap=0.0, **kw):
    say(p.name)
    out, lse = run_gpu_paged(p, out_fill=float("nan"), alibi=alibi, softcap=softcap, **kw)
    ref_o, ref_l = run_oracle_paged(p, alibi=alibi, softcap=softcap)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


# decode steps, a chunk over a context, a one-key sequence, a prefill spanning several
# query blocks and tiles, a sequence without queries, more queries than keys, no keys
Q_LENS = [1, 37, 1, 130, 0, 5, 3]
K_LENS = [300, 200, 1, 130, 50, 3, 0]


def test_mixed_batch_paged_bf16():
    check(synth.paged_config("v1"))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp16", 128), ("fp16", 64)])
@pytest.mark.parametrize("kind", ["none", "causal", "window"])
@pytest.mark.parametrize("page_size", [0, 1, 16, 128])
def test_dtypes_masks_pages(dtype, d, kind, page_size):
    p = synth.make_paged_problem(f"varlen {dtype} d{d} {kind} page{page_size}", Q_LENS, K_LENS, 8, 2, d, dtype,
                                 kind, 300 + d + page_size, page_size=page_size, window_left=45)
    check(p)


@pytest.mark.parametrize("page_size", [0, 16])
@pytest.mark.parametrize("kind", ["causal", "window", "none"])
def test_two_source(kind, page_size):
    # the last sequence has fewer keys than queries: no cached/new split, rows masked
    q_lens, k_lens = [1, 37, 1, 130, 0, 64, 3], [300, 200, 1, 130, 50, 64, 2]
    p = synth.make_paged_problem(f"two-source {kind} page{page_size}", q_lens, k_lens, 8, 2, 128, "bf16", kind,
                                 410 + page_size, page_size=page_size, two_source=True, window_left=70)
    check(p)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (4, 4), (32, 1), (128, 1)])
def test_gqa_group_sizes(Hq, Hkv):
    p = synth.make_paged_problem(f"varlen GQA {Hq}/{Hkv}", [1, 19, 70, 2], [1000, 19, 333, 65], Hq, Hkv, 128,
                                 "bf16", "causal", 500 + Hq, page_size=32)
    check(p)


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_forced_splits(splits):
    import masked_flashattention_forward_amd as mfa
    p = synth.make_paged_problem(f"varlen forced splits {splits}", Q_LENS, K_LENS, 8, 2, 128, "bf16", "causal",
                                 600 + splits, page_size=16)
    mfa.set_debug(force_splits=splits)
    try:
        check(p)
    finally:
        mfa.set_debug()


SLOPES8 = [2.0 ** -(i + 1) for i in range(8)]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("kind", ["none", "causal", "window"])
@pytest.mark.parametrize("mods", ["alibi", "softcap", "both"])
def test_score_modifiers(dtype, d, kind, mods):
    """ALiBi and softcap on every sequence's own positions, on the prefill-type and the
    decode-type kernels of one batch (N(0,1) inputs, a cap that bends the scores)."""
    p = synth.make_paged_problem(f"varlen {mods} {kind} {dtype} d{d}", Q_LENS, K_LENS, 8, 2, d, dtype, kind,
                                 800 + d, page_size=16, window_left=45)
    check(p, alibi=SLOPES8 if mods != "softcap" else None, softcap=0.8 if mods != "alibi" else 0.0)


@pytest.mark.parametrize("form", ["two_source", "split"])
def test_score_modifiers_two_source_and_split(form):
    import masked_flashattention_forward_amd as mfa
    q_lens, k_lens = [1, 37, 1, 130, 0, 64, 3], [300, 200, 1, 130, 50, 64, 2]
    p = synth.make_paged_problem(f"varlen modifiers {form}", q_lens, k_lens, 8, 2, 128, "bf16", "causal", 820,
                                 page_size=16, two_source=form == "two_source")
    mfa.set_debug(force_splits=3 if form == "split" else 0)
    try:
        check(p, alibi=SLOPES8, softcap=1.3)
    finally:
        mfa.set_debug()


def test_decode_batch_splits_automatically():
    """Few long decode sequences: too few work units, so the key range is split."""
    p = synth.make_paged_problem("varlen decode 6 x long", [1] * 6, [9000, 4097, 1, 12000, 640, 7000], 32, 8,
                                 128, "bf16", "causal", 700, page_size=16)
    check(p)


def test_understated_max_seqlen_k_is_only_a_hint():
    p = synth.make_paged_problem("varlen max_seqlen_k hint 1", [1, 3], [5000, 4000], 8, 2, 128, "bf16",
                                 "causal", 701, page_size=64)
    check(p, max_seqlen_k=1)


def test_matches_the_batched_forward_on_equal_lengths():
    """B equal-length sequences with pages in order give the single-batch forward's
    result: the same tiles in the same order, so the same bits."""
    import torch
    import masked_flashattention_forward_amd as mfa
    from helpers import to_device
    B, L, Hq, Hkv, d, ps = 3, 300, 8, 2, 128, 16
    p = synth.make_paged_problem("varlen vs batched", [L] * B, [L] * B, Hq, Hkv, d, "bf16", "causal", 702,
                                 page_size=ps, spare_pages=0)
    say(p.name)
    pages = (L + ps - 1) // ps
    k = to_device(p.k, "bf16").reshape(B, pages * ps, Hkv, d)
    v = to_device(p.v, "bf16").reshape(B, pages * ps, Hkv, d)
    table = torch.arange(B * pages, dtype=torch.int32, device="cuda").reshape(B, pages)
    q = to_device(p.q, "bf16")
    cu = torch.from_numpy(p.cu_seqlens_q).cuda()
    o1, l1 = mfa.attn_fwd_varlen(q, k.reshape(B * pages, ps, Hkv, d), v.reshape(B * pages, ps, Hkv, d), cu, cu,
                                 max_seqlen_q=L, max_seqlen_k=L, block_table=table)
    qb = q.reshape(B, L, Hq, d).transpose(1, 2).contiguous()
    kb = k[:, :L].transpose(1, 2).contiguous()
    vb = v[:, :L].transpose(1, 2).contiguous()
    o2, l2 = mfa.attn_fwd(qb, kb, vb)
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(B, L, Hq, d).transpose(1, 2), o2)
    assert torch.equal(l1.reshape(B, L, Hq).transpose(1, 2), l2)


@pytest.mark.slow
def test_serving_batch_sampled_sequences():
    p = synth.paged_config("serve")
    say(p.name)
    out, lse = run_gpu_paged(p, out_fill=float("nan"))
    seqs = [0, 3, 4, 17, 40, 63]   # two prefill chunks and four decode steps
    ref_o, ref_l = run_oracle_paged(p, seqs=seqs)
    compare(p, out, lse, ref_o, ref_l, label=p.name + " (sampled sequences)")
    assert not np.isnan(out).any() and not np.isnan(lse).any()


@pytest.mark.slow
def test_serving_batch_with_modifiers_sampled():
    """The serving batch with ALiBi + softcap as bench.py times it, on sampled sequences."""
    p = synth.paged_config("serve")
    say(p.name + " + ALiBi + softcap 30")
    alibi = synth.alibi_slopes(p.Hq)
    out, lse = run_gpu_paged(p, out_fill=float("nan"), alibi=alibi, softcap=30.0)
    seqs = [0, 3, 4, 17, 40, 63]
    ref_o, ref_l = run_oracle_paged(p, seqs=seqs, alibi=alibi, softcap=30.0)
    compare(p, out, lse, ref_o, ref_l, label=p.name + " + modifiers (sampled sequences)")
    assert not np.isnan(out).any() and not np.isnan(lse).any()


@pytest.mark.parametrize("G", [1, 8, 32])
def test_decode_type_boundary(G):
    """Sequences with exactly 32 query rows per KV head run on the decode kernel, one row
    more on the prefill kernel; both next to each other in one call."""
    Hkv = 2
    q_lens = [32 // G, 32 // G + 1, 1, 32 // G]
    k_lens = [900, 900, 2000, 70]
    p = synth.make_paged_problem(f"varlen decode/prefill boundary G{G}", q_lens, k_lens, G * Hkv, Hkv, 128, "bf16",
                                 "causal", 800 + G, page_size=16)
    check(p)
