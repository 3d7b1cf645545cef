"""Resident prefill workgroups: when a prefill grid of a key-position mask (none, causal,
window) has more query blocks than the GPU holds at once, attn_fwd launches only the
resident workgroups and each takes several blocks (the blocks of its XCD's list in zigzag
rounds). The cases have more blocks than two workgroups per CU on 256 CUs and cover the
three position kinds, both head dims and both half types, with ragged query blocks (Lq
not a multiple of the block); a dense and a gathered top-k case of the same size check
the one-workgroup-per-block launch those kinds keep. The outputs start as NaN, so a block
that no workgroup takes fails; the first and last row of every query block, over every
(batch, head), are compared with the oracle, and a second call must give the same bits."""
import numpy as np
import pytest

import synth
from helpers import compare, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

RESIDENT = 2 * 256  # two workgroups per CU on 256 CUs: every grid below is larger


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


def problems():
    rng = np.random.default_rng(4301)
    dense = np.where(rng.random((1000, 1000)) < 0.2, -np.inf, rng.standard_normal((1000, 1000))).astype(np.float32)
    return [
        synth.make_problem("resident causal bf16 d128 4x16 2000", 4, 16, 16, 2000, 2000, 128, "bf16", "causal", 4201),
        synth.make_problem("resident none fp16 d64 GQA 2x32/8 2100x3000", 2, 32, 8, 2100, 3000, 64, "fp16", "none",
                           4202),
        synth.make_problem("resident window bf16 d64 4x16 2048", 4, 16, 16, 2048, 2048, 64, "bf16", "window", 4203,
                           window_left=300),
        synth.make_problem("resident dense fp16 d128 8x16 1000", 8, 16, 16, 1000, 1000, 128, "fp16", "dense", 4204,
                           mask=dense),
        synth.make_problem("resident top-k bf16 d128 2x16 4000", 2, 16, 16, 4000, 4000, 128, "bf16", "topk", 4205,
                           keep_k=1024, with_zero_hold=True),
    ]


@pytest.mark.parametrize("idx", range(5))
def test_resident_workgroups(idx):
    import masked_flashattention_forward_amd as mfa
    p = problems()[idx]
    plan = mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, p.mask_kind, p.window_left, p.keep_k,
                    synth.DTYPE_CODES[p.dtype])
    assert plan["path"] == "mfma_prefill" and plan["splits"] == 1 and plan["grid"] > RESIDENT, plan
    say(f"{p.name}: {plan['grid']} query blocks")
    out, lse = run_gpu(p, out_fill=float("nan"))
    assert not np.isnan(out).any() and not np.isnan(lse).any(), f"{p.name}: a block was not computed"
    qpb = plan["block_m"] // (p.Hq // p.Hkv)
    rows = sorted({r for qb0 in range(0, p.Lq, qpb) for r in (qb0, min(p.Lq, qb0 + qpb) - 1)})
    ref_o, ref_l = run_oracle(p, rows=rows)
    compare(p, out, lse, ref_o, ref_l, rows=rows, label=f"{p.name}, first and last row of every block")
    out2, lse2 = run_gpu(p, out_fill=float("nan"))
    np.testing.assert_array_equal(out2, out, err_msg=f"{p.name}: second call differs")
    np.testing.assert_array_equal(lse2, lse, err_msg=f"{p.name}: second call differs (LSE)")


def test_two_streams_at_once():
    """Resident grids of two calls launched on two streams with no ordering between them
    (the library takes no workspace for them, so nothing serialises the calls): the
    workgroups of one grid wait for the other's slots, and every block is still computed
    once, with the bits of the calls run alone."""
    import torch
    import masked_flashattention_forward_amd as mfa
    from helpers import to_device
    ps = problems()[:3]
    dev = []
    for p in ps:
        q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
        dev.append((p, q, k, v))

    def run(p, q, k, v, stream=None):
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
            lse = torch.full((p.B, p.Hq, p.Lq), float("nan"), dtype=torch.float32, device="cuda")
        mfa.attn_fwd(q, k, v, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left, out=out, lse=lse,
                     stream=stream)
        return out, lse

    ref = []
    for p, q, k, v in dev:
        o, l = run(p, q, k, v)
        torch.cuda.synchronize()
        ref.append((o.view(torch.int16).cpu().numpy(), l.cpu().numpy()))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rnd in range(3):
        say(f"resident grids on two streams at once, round {rnd}")
        torch.cuda.synchronize()
        res = [run(*d, stream=s1 if i % 2 == 0 else s2) for i, d in enumerate(dev)]
        torch.cuda.synchronize()
        for (p, *_), (o, l), (o_ref, l_ref) in zip(dev, res, ref):
            np.testing.assert_array_equal(o.view(torch.int16).cpu().numpy(), o_ref,
                                          err_msg=f"{p.name}: output differs on two streams")
            np.testing.assert_array_equal(l.cpu().numpy(), l_ref, err_msg=f"{p.name}: LSE differs on two streams")
    print("[resident] three resident grids on two streams at once, three rounds: bit-identical", flush=True)
