"""Randomised shapes on the GPU against the fp64 oracle: forward (attn_fwd) and backward
(attn_bwd) over seeded draws of batch, head counts and grouping, lengths (Lq above, equal to
and below Lk, one-row and one-key cases), head dim, dtype and mask kind with its parameters.
Every draw is printed before it runs, so a failure names its case."""
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
