"""The per-GPU workspace arena that holds every call's temporary memory (top-k ranks,
thresholds, sorted key chunks and kept-key lists; split-KV partials).

Calls on two streams enqueued back to back with no host synchronisation, each needing
temporary memory, must give the same bits as the same calls run one at a time: a call on
the other stream may only reuse the block once the previous user's work is done. A
sequence small / large / small (the large call may grow the block) must stay exact too.
Inputs are seeded synthetic problems of the c5 (top-k) and c3 decode kinds at reduced
sizes."""
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


class Call:
    """Device inputs of one problem and an attn_fwd call on a given stream (not synchronised)."""

    def __init__(self, p):
        import torch
        self.p = p
        self.q, self.k, self.v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
        self.zh = None if p.zero_hold is None else torch.from_numpy(p.zero_hold).cuda()
        self.out = torch.full(self.q.shape, float("nan"), dtype=self.q.dtype, device="cuda")
        self.lse = torch.full((p.B, p.Hq, p.Lq), float("nan"), dtype=torch.float32, device="cuda")

    def __call__(self, stream=None):
        import masked_flashattention_forward_amd as mfa
        p = self.p
        mfa.attn_fwd(self.q, self.k, self.v, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left,
                     zero_hold=self.zh, keep_k=p.keep_k, out=self.out, lse=self.lse, stream=stream)

    def result(self):
        import torch
        o = self.out.view(torch.int16) if self.out.element_size() == 2 else self.out
        return o.cpu().numpy().copy(), self.lse.cpu().numpy().copy()


def problems():
    return [
        synth.make_problem("arena top-k 2x8 3000", 2, 8, 8, 3000, 3000, 128, "bf16", "topk", 4101, keep_k=700,
                           with_zero_hold=True),
        synth.make_problem("arena decode 4x16/4 1x20000", 4, 16, 4, 1, 20000, 128, "bf16", "causal", 4102),
        synth.make_problem("arena top-k 1x16 4096", 1, 16, 16, 4096, 4096, 128, "bf16", "topk", 4103, keep_k=1024,
                           with_zero_hold=True),
        synth.make_problem("arena decode 8x32/8 1x9000", 8, 32, 8, 1, 9000, 64, "fp16", "causal", 4104),
    ]


def test_two_streams_share_the_arena():
    import torch
    import masked_flashattention_forward_amd as mfa
    calls = [Call(p) for p in problems()]
    for c in calls:
        plan = mfa.plan(c.p.B, c.p.Hq, c.p.Hkv, c.p.Lq, c.p.Lk, c.p.d, c.p.mask_kind, c.p.window_left, c.p.keep_k,
                        synth.DTYPE_CODES[c.p.dtype])
        assert plan["workspace_bytes"] > 0, (c.p.name, plan)
    # one at a time
    ref = []
    for c in calls:
        say(f"alone: {c.p.name}")
        c()
        torch.cuda.synchronize()
        ref.append(c.result())
        c.out.fill_(float("nan"))
        c.lse.fill_(float("nan"))
    torch.cuda.synchronize()
    # alternating streams, enqueued back to back, three rounds
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rnd in range(3):
        say(f"two streams, round {rnd}")
        for i, c in enumerate(calls):
            c(stream=s1 if i % 2 == 0 else s2)
        torch.cuda.synchronize()
        for c, (o_ref, l_ref) in zip(calls, ref):
            o, l = c.result()
            np.testing.assert_array_equal(o, o_ref, err_msg=f"{c.p.name}: output differs on two streams")
            np.testing.assert_array_equal(l, l_ref, err_msg=f"{c.p.name}: LSE differs on two streams")
            c.out.fill_(float("nan"))
            c.lse.fill_(float("nan"))
        torch.cuda.synchronize()
    print("[arena] four calls on two streams, three rounds: bit-identical to one at a time", flush=True)


def test_small_large_small():
    import torch
    small = Call(synth.make_problem("arena small top-k", 1, 4, 4, 700, 700, 64, "bf16", "topk", 4105, keep_k=100,
                                    with_zero_hold=True))
    large = Call(synth.make_problem("arena large top-k", 2, 16, 16, 12000, 12000, 64, "bf16", "topk", 4106,
                                    keep_k=2000, with_zero_hold=True))
    ref = []
    for c in (small, large):
        c()
        torch.cuda.synchronize()
        ref.append(c.result())
    for rnd in range(2):
        say(f"small / large / small, round {rnd}")
        for c in (small, large, small):
            c.out.fill_(float("nan"))
            c()
        torch.cuda.synchronize()
        for c, (o_ref, l_ref) in zip((small, large), ref):
            o, l = c.result()
            np.testing.assert_array_equal(o, o_ref, err_msg=f"{c.p.name}: output differs")
            np.testing.assert_array_equal(l, l_ref, err_msg=f"{c.p.name}: LSE differs")
    print("[arena] small / large / small: bit-identical", flush=True)
