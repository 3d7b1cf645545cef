"""attn_fwd_noalloc (the entry point that takes its temporary memory from the library's
fixed per-GPU scratch) against attn_fwd through the C ABI: the same kernels run, so the
results must be bit-identical, on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents). The cases use every kind of temporary
memory: split-KV partials (decode path), top-k ranks, thresholds, sorted key chunks and
kept-key lists, and dense-mask tile flags. A call that needs more than the fixed size is
refused before any work."""
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


def both(p):
    """(attn_fwd, attn_fwd_noalloc) outputs and LSE on device copies of p's inputs."""
    import torch
    import masked_flashattention_forward_amd as mfa
    q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    mask = None if p.mask is None else torch.from_numpy(p.mask).cuda()
    zh = None if p.zero_hold is None else torch.from_numpy(p.zero_hold).cuda()
    res = []
    for noalloc in (False, True):
        out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
        lse = torch.full((p.B, p.Hq, p.Lq), float("nan"), dtype=torch.float32, device="cuda")
        mfa.attn_fwd(q, k, v, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left,
                     mask=mask if p.mask_kind == "dense" else None, zero_hold=zh, keep_k=p.keep_k, out=out, lse=lse,
                     noalloc=noalloc)
        torch.cuda.synchronize()
        res.append((out.view(torch.int16).cpu().numpy() if out.element_size() == 2 else out.cpu().numpy(),
                    lse.cpu().numpy()))
    return res


def check_equal(p, label):
    import masked_flashattention_forward_amd as mfa
    say(label)
    plan = mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, p.mask_kind, p.window_left, p.keep_k,
                    synth.DTYPE_CODES[p.dtype])
    assert 0 < plan["workspace_bytes"] <= mfa.NOALLOC_MAX_WORKSPACE, plan
    (o1, l1), (o2, l2) = both(p)
    assert not np.isnan(l2).all()
    np.testing.assert_array_equal(o2, o1, err_msg=f"{label}: output differs from attn_fwd")
    np.testing.assert_array_equal(l2, l1, err_msg=f"{label}: LSE differs from attn_fwd")
    print(f"[noalloc] {label}: bit-identical to attn_fwd (workspace {plan['workspace_bytes']} bytes)", flush=True)


# (first, second): the second call of each pair is smaller
PAIRS = [
    # top-k with kept-key lists and sorted chunks, then a smaller top-k
    (("topk big", 2, 8, 4, 700, 1500, 128, "bf16", "topk", 1401, dict(keep_k=200, with_zero_hold=True)),
     ("topk small", 1, 4, 2, 77, 203, 64, "fp16", "topk", 1402, dict(keep_k=17, with_zero_hold=True))),
    # split-KV decode partials, then a smaller decode
    (("decode big", 4, 32, 8, 1, 8192, 128, "bf16", "causal", 1403, {}),
     ("decode small", 2, 8, 2, 1, 3000, 128, "bf16", "causal", 1404, {})),
    # dense-mask tile flags (built from 2048 keys up), then smaller flags
    (("dense big", 4, 32, 8, 16, 2900, 128, "bf16", "dense", 1405,
      dict(mask=synth.window_dense_mask(16, 2900, 2884, 300))),
     ("dense small", 1, 4, 2, 9, 2100, 64, "bf16", "dense", 1406,
      dict(mask=synth.window_dense_mask(9, 2100, 2091, 200)))),
]


@pytest.mark.parametrize("pair", PAIRS, ids=["topk", "decode", "dense"])
def test_noalloc_matches_attn_fwd_twice(pair):
    for name, B, Hq, Hkv, Lq, Lk, d, dtype, kind, seed, kw in pair:
        p = synth.make_problem(f"noalloc {name}", B, Hq, Hkv, Lq, Lk, d, dtype, kind, seed, **kw)
        check_equal(p, p.name)


def test_noalloc_refuses_a_plan_above_the_fixed_scratch():
    """Top-k over 64 (batch, head) pairs of 16384 keys needs more temporary memory than
    the fixed scratch holds: refused with MI_ATTN_EUNSUPPORTED, nothing enqueued."""
    import torch
    import masked_flashattention_forward_amd as mfa
    B, H, Lq, Lk, d = 4, 16, 4096, 16384, 64
    plan = mfa.plan(B, H, H, Lq, Lk, d, "topk", keep_k=2048, dtype=mfa.BF16)
    assert plan["workspace_bytes"] > mfa.NOALLOC_MAX_WORKSPACE, plan
    q = torch.zeros((B, H, Lq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Lk, d), dtype=torch.bfloat16, device="cuda")
    zh = torch.zeros((B, H, Lk), dtype=torch.float32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(mfa.MiAttnError) as e:
        mfa.attn_fwd(q, k, k, mask_kind="topk", zero_hold=zh, keep_k=2048, out=out, noalloc=True)
    assert e.value.code == mfa.EUNSUPPORTED and "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call wrote its output"
