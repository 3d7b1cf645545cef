"""GPU parity of attn_bwd (dq, dk, dv) against the fp64 oracle (oracle/backward.py).

The GPU forward writes out and lse; the backward consumes them with a seeded output
gradient. The oracle differentiates the exact forward of the stored (rounded) inputs.

Tolerance, derived from the arithmetic of the kernels (u = 2^-8 for bf16, 2^-11 for
fp16, the unit roundoff of the input type): products take 16-bit operands with fp32
accumulation, so the errors that matter are the roundings to the input type of
  - the forward output O (its P rounded, then O itself): |dO_i| . (sum_j P_ij |v_j| + |O_i|) u
    bounds the error of D_i = rowsum(dout * out) computed from that output;
  - P before dv = P^T dO:                       u sum_i P_ij |dO_ic|
  - dS = P (dP - D) before dq and dk:           P_ij |dD_i| + u |dS_ij| per element
  - the gradients themselves:                   u |g|.
Each rounding also carries an absolute part, eta = half the smallest subnormal step of the
type (2^-25 for fp16, 2^-134 for bf16): tiny P, dS and gradient values land in the
subnormal range or flush to zero, which a relative bound alone does not cover.
Each element must sit within twice the sum of these bounds (fp32 accumulation and the
exp2/LSE errors, ~1e-6 relative, are far below u). The bound is worst-case; a statistical
check adds that the relative RMS error of each gradient stays below 4u (rounding gives
about u), which a dropped term or a wrong index would far exceed.
"""
import numpy as np
import pytest

import synth
from helpers import say, to_device

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
ETA = {"bf16": 2.0 ** -134, "fp16": 2.0 ** -25}


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


def dout_for(p, seed):
    return synth.to_storage(synth.draw(seed, [(p.B, p.Hq, p.Lq, p.d)])[0], p.dtype)


def run_gpu_bwd(p, dout_s, *, no_skip=False):
    """attn_fwd then attn_bwd on the GPU; returns (dq, dk, dv) as fp64 arrays."""
    import torch
    import masked_flashattention_forward_amd as mfa
    q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    dout = to_device(dout_s, p.dtype)
    mask = None if p.mask is None else torch.from_numpy(p.mask).cuda()
    zh = None if p.zero_hold is None else torch.from_numpy(p.zero_hold).cuda()
    kw = dict(scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left, mask=mask, zero_hold=zh,
              keep_k=p.keep_k)
    out, lse = mfa.attn_fwd(q, k, v, **kw)
    grads = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    mfa.set_debug(no_skip=no_skip)
    try:
        mfa.attn_bwd(q, k, v, out, lse, dout, dq=grads[0], dk=grads[1], dv=grads[2], **kw)
        torch.cuda.synchronize()
    finally:
        mfa.set_debug()
    return tuple(g.to(torch.float32).cpu().numpy().astype(np.float64) for g in grads)


def oracle_with_bounds(p, dout64, heads=None):
    """Oracle gradients and the per-element bounds of the module docstring. With heads =
    [(b, g), ...] only those (batch, KV head) pairs are computed (the rest is NaN)."""
    from oracle import mask_matrix
    from oracle.backward import softmax_backward_terms
    u, eta = U[p.dtype], ETA[p.dtype]
    q, k, v = p.f64("q"), p.f64("k"), p.f64("v")
    mask = None if p.mask is None else p.mask.astype(np.float64)
    zh = None if p.zero_hold is None else p.zero_hold.astype(np.float64)
    G = p.Hq // p.Hkv
    ref = [np.full(x.shape, np.nan) for x in (q, k, v)]
    bnd = [np.full(x.shape, np.nan) for x in (q, k, v)]
    pairs = heads if heads is not None else [(b, g) for b in range(p.B) for g in range(p.Hkv)]
    s = abs(p.scale64)
    for b, g in pairs:
        A = mask_matrix(p.mask_kind, p.Lq, p.Lk, window_left=p.window_left, dense=mask,
                        zh_row=None if zh is None else zh[b, g], keep_k=p.keep_k)
        kb, vb = k[b, g], v[b, g]
        for x in (ref, bnd):
            x[1][b, g] = 0.0
            x[2][b, g] = 0.0
        for h in range(g * G, (g + 1) * G):
            P, dZ = softmax_backward_terms(q[b, h], kb, vb, dout64[b, h], p.scale64, A)
            do = dout64[b, h]
            ref[0][b, h] = p.scale64 * (dZ @ kb)
            ref[1][b, g] += p.scale64 * (dZ.T @ q[b, h])
            ref[2][b, g] += P.T @ do
            dD = u * (np.abs(do) * (P @ np.abs(vb) + np.abs(P @ vb))).sum(axis=1)
            E = P * dD[:, None] + u * np.abs(dZ) + eta
            bnd[0][b, h] = s * (E @ np.abs(kb))
            bnd[1][b, g] += s * (E.T @ np.abs(q[b, h]))
            bnd[2][b, g] += (u * P + eta).T @ np.abs(do)
    for r, e in zip(ref, bnd):
        e += u * np.abs(r) + eta
    return ref, bnd


def compare_grads(p, got, ref, bnd, label, dead_rows=None):
    u = U[p.dtype]
    for name, g, r, e in zip(("dq", "dk", "dv"), got, ref, bnd):
        sel = ~np.isnan(r)
        assert sel.any()
        gs, rs, es = g[sel], r[sel], e[sel]
        assert np.isfinite(gs).all(), f"{label}: non-finite {name}"
        err = np.abs(gs - rs)
        ratio = float((err / (2.0 * es + 1e-30)).max())
        rms = float(np.sqrt(np.mean((gs - rs) ** 2)) / max(np.sqrt(np.mean(rs ** 2)), 1e-30))
        print(f"[parity] {label} {name}: max|err|={err.max():.3e} max err/bound={ratio:.3f} "
              f"rel rms={rms:.2e} (limit {4 * u:.1e})", flush=True)
        assert ratio <= 1.0, f"{label}: {name} error beyond its bound ({ratio:.3f})"
        if np.sqrt(np.mean(rs ** 2)) > 0:
            assert rms <= 4 * u, f"{label}: {name} relative RMS error {rms:.2e}"
    if dead_rows is not None:
        assert np.all(got[0][dead_rows] == 0.0), f"{label}: rows that see no key must get dq = 0"


def check(p, seed, label=None, **kw):
    label = label or p.name
    say(label)
    dout_s = dout_for(p, seed)
    got = run_gpu_bwd(p, dout_s, **kw)
    ref, bnd = oracle_with_bounds(p, synth.storage_to_f64(dout_s, p.dtype))
    compare_grads(p, got, ref, bnd, label)
    return got


def dead_row_mask(Lq, Lk, seed):
    rng = np.random.default_rng(seed)
    m = rng.standard_normal((Lq, Lk)).astype(np.float32)
    m[rng.random(m.shape) < 0.4] = -np.inf
    m[min(3, Lq - 1)] = -np.inf          # a row that sees no key
    m[:, Lk // 3: Lk // 3 + 70] = -np.inf  # keys no row sees
    return m


# (dtype, d, B, Hq, Hkv, Lq, Lk): MHA and GQA/MQA (up to 128 query heads per KV head, the
# most attn_bwd takes), ragged tails against the 32-row, 64-key and 128-key tiles, Lq below,
# equal to and above Lk, one-row decode
SHAPES = [("bf16", 128, 2, 4, 2, 77, 203), ("fp16", 64, 2, 4, 2, 77, 203), ("bf16", 64, 1, 2, 2, 130, 130),
          ("fp16", 128, 1, 8, 1, 100, 100), ("bf16", 128, 2, 6, 2, 1, 300), ("bf16", 128, 1, 4, 4, 300, 100),
          ("fp16", 128, 1, 16, 1, 33, 260), ("bf16", 128, 1, 128, 1, 5, 150)]
KINDS = ["none", "causal", "window", "dense", "topk"]


def shape_id(s):
    return f"{s[0]}-d{s[1]}-B{s[2]}-H{s[3]}x{s[4]}-{s[5]}x{s[6]}"


@pytest.mark.parametrize("shape", SHAPES, ids=shape_id)
@pytest.mark.parametrize("kind", KINDS)
def test_backward_matches_oracle(shape, kind):
    dtype, d, B, Hq, Hkv, Lq, Lk = shape
    p = synth.make_problem(f"bwd {kind} {shape_id(shape)}", B, Hq, Hkv, Lq, Lk, d, dtype, kind, 1500 + d + Lq,
                           window_left=41, keep_k=29, with_zero_hold=kind == "topk",
                           mask=dead_row_mask(Lq, Lk, 7) if kind == "dense" else None)
    check(p, 1600 + Lk)


@pytest.mark.parametrize("kind", ["causal", "window", "dense", "topk"])
def test_skipped_tiles_contribute_nothing(kind):
    """Visiting every tile (the no-skip debug switch) gives bit-identical gradients."""
    p = synth.make_problem(f"bwd no-skip {kind}", 1, 4, 2, 150, 420, 128, "bf16", kind, 1700, window_left=50,
                           keep_k=40, with_zero_hold=kind == "topk",
                           mask=dead_row_mask(150, 420, 9) if kind == "dense" else None)
    say(p.name)
    dout_s = dout_for(p, 1701)
    a = run_gpu_bwd(p, dout_s)
    b = run_gpu_bwd(p, dout_s, no_skip=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_rows_that_see_no_key_get_zero_dq():
    # causal with Lq > Lk: the first Lq - Lk rows sit before every key
    p = synth.make_problem("bwd rows before every key", 1, 2, 1, 90, 40, 64, "bf16", "causal", 1800)
    say(p.name)
    dout_s = dout_for(p, 1801)
    got = run_gpu_bwd(p, dout_s)
    ref, bnd = oracle_with_bounds(p, synth.storage_to_f64(dout_s, p.dtype))
    dead = np.zeros(got[0].shape, dtype=bool)
    dead[:, :, : p.Lq - p.Lk] = True
    compare_grads(p, got, ref, bnd, p.name, dead_rows=dead)


def test_negative_scale():
    p = synth.make_problem("bwd negative scale", 1, 4, 2, 70, 150, 128, "bf16", "causal", 1900, scale=-0.09)
    check(p, 1901)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_large_logits(dtype):
    """Inputs 4x larger: sharp softmax rows (P near one-hot)."""
    p = synth.make_problem(f"bwd large logits {dtype}", 1, 4, 2, 96, 256, 64, dtype, "causal", 2000, mult=4.0)
    check(p, 2001)


BENCH_SAMPLES = {"c4_d128_bf16": [(0, 0), (3, 15)], "c4_d64_bf16": [(1, 7)], "c3p": [(0, 0), (7, 7)]}


@pytest.mark.slow
@pytest.mark.parametrize("name", list(BENCH_SAMPLES))
def test_backward_full_size_sampled(name):
    """The backward workloads bench.py times, at full size and in the same call, against
    the oracle on sampled (batch, KV head) pairs (every query row of their heads)."""
    p = synth.config(name)
    say(f"bwd {name}: {p.name}")
    dout_s = dout_for(p, 2100)
    got = run_gpu_bwd(p, dout_s)
    ref, bnd = oracle_with_bounds(p, synth.storage_to_f64(dout_s, p.dtype), heads=BENCH_SAMPLES[name])
    compare_grads(p, got, ref, bnd, f"{name} (sampled heads)")


@pytest.mark.parametrize("kind,Lq,Lk,extra", [
    ("causal", 1, 1, {}),                      # one row, one key
    ("none", 5, 1, {}),                        # a single key for every row
    ("window", 40, 90, {"window_left": 0}),    # each row sees only its own position
    ("dense", 9, 33, {"mask": "all -inf"}),    # every row dead: all gradients zero
    ("topk", 64, 64, {"keep_k": 1}),           # one kept key per row
])
def test_backward_edge_cases(kind, Lq, Lk, extra):
    mask = None
    if extra.get("mask") == "all -inf":
        mask = np.full((Lq, Lk), -np.inf, dtype=np.float32)
    p = synth.make_problem(f"bwd edge {kind} {Lq}x{Lk} {extra}", 2, 4, 2, Lq, Lk, 128, "bf16", kind, 2200 + Lq,
                           window_left=extra.get("window_left", 0), keep_k=extra.get("keep_k", 0),
                           with_zero_hold=kind == "topk", mask=mask)
    got = check(p, 2201)
    if mask is not None:
        for g in got:
            assert np.all(g == 0.0)
