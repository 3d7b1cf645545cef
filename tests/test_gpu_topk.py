"""GPU dynamic top-k selection against the oracle: ranks, thresholds and kept sets must
match bit for bit (flash-sparse-attention issue #11 page, "Current Status": the mask
computation has to agree exactly, position match 1.0)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check_topk(zh: np.ndarray, Lq: int, keep_k: int, causal: bool, label: str, heads=None):
    import torch
    import masked_flashattention_forward_amd as mfa
    say(label)
    B, H, Lk = zh.shape
    rank, tau, bits = mfa.dynamic_mask_topk(torch.from_numpy(zh).cuda(), Lq, keep_k, causal=causal,
                                            with_bits=True)
    torch.cuda.synchronize()
    rank, tau = rank.cpu().numpy(), tau.cpu().numpy()
    bits = bits.cpu().numpy().view(np.uint32)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in heads:
        z = zh[b, h].astype(np.float64)
        r_ref = oracle.topk_rank_ref(z)
        np.testing.assert_array_equal(rank[b, h], r_ref, err_msg=f"{label} rank b{b} h{h}")
        t_ref = oracle.topk_tau_ref(r_ref, Lq, keep_k, causal=causal)
        np.testing.assert_array_equal(tau[b, h], t_ref, err_msg=f"{label} tau b{b} h{h}")
        kept = oracle.topk_kept_ref(z, Lq, keep_k, causal=causal)
        np.testing.assert_array_equal(bits[b, h], oracle.pack_keep_bits(kept), err_msg=f"{label} bits b{b} h{h}")
    print(f"[topk] {label}: kept sets bit-exact on {len(heads)} heads", flush=True)


@pytest.mark.parametrize("Lq,Lk,keep_k", [(4, 4, 2), (77, 203, 17), (203, 203, 1), (50, 300, 300),
                                          (300, 120, 7), (1, 5000, 64), (64, 9000, 100)])
@pytest.mark.parametrize("causal", [True, False])
def test_topk_random_with_ties(Lq, Lk, keep_k, causal):
    rng = np.random.default_rng(Lq * 7 + Lk)
    zh = (rng.integers(-4, 5, size=(2, 3, Lk)) * 0.5).astype(np.float32)
    zh[rng.random(zh.shape) < 0.1] = -0.0
    check_topk(zh, Lq, keep_k, causal, f"ties Lq{Lq} Lk{Lk} k{keep_k} causal{causal}")


def test_topk_minimal_golden():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "minimal_topk_example.json")))
    for case in g["cases"]:
        zh = np.array([float(x) for x in case["zero_hold"]], dtype=np.float32)[None, None]
        check_topk(zh, case["Lq"], case["keep_k"], True, "minimal: " + case["name"])


def test_topk_c5_full_size():
    """Every (batch, head) of the top-k workload at its full size."""
    p = synth.config("c5")
    check_topk(p.zero_hold, p.Lq, p.keep_k, True, "c5 zero_hold [2,16,4096] k=1024, all 32 heads")


@pytest.mark.parametrize("Lk", [8192, 8193, 16391, 32768, 40001, 65536])
@pytest.mark.parametrize("causal", [True, False])
def test_topk_long_caches(Lk, causal):
    """At 8192 keys the ranks come from the sixteen sorted 512-key chunks staged in LDS
    together (the largest staging); past 8192 keys the chunks are merged into sorted runs
    of 8192 keys before the ranks are counted: ranks, thresholds and keep bits bit-exact,
    with long runs of tied values and -0.0 beside +0.0, including a partial last run and a
    partial last chunk."""
    rng = np.random.default_rng(Lk + int(causal))
    zh = rng.standard_normal((1, 2, Lk)).astype(np.float32)
    zh[0, 0, rng.random(Lk) < 0.4] = np.float32(0.75)
    zh[0, 1, : Lk // 3] = -0.0
    zh[0, 1, Lk // 3: Lk // 2] = 0.0
    Lq = 40
    check_topk(zh, Lq, 3000, causal, f"long cache Lk{Lk} causal{int(causal)}")


def test_topk_attention_at_the_largest_cache():
    """Top-k attention over 65536 keys, the largest cache the top-k mask takes (eight sorted
    runs), for the last 64 query positions, against the oracle."""
    from helpers import compare, run_gpu, run_oracle
    p = synth.make_problem("top-k attention Lk 65536", 1, 4, 2, 64, 65536, 128, "bf16", "topk", 1602, keep_k=2000,
                           with_zero_hold=True)
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


def test_topk_attention_over_a_long_cache():
    """Top-k attention (kept-key lists) over 20000 keys, against the oracle."""
    from helpers import compare, run_gpu, run_oracle
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem("top-k attention Lk 20000", 1, 4, 2, 300, 20000, 128, "bf16", "topk", 1601, keep_k=700,
                           with_zero_hold=True)
    assert mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, "topk", keep_k=p.keep_k)["topk_list_cap"] > 0
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)
