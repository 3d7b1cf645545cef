"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by
element, on seeded inputs. Small shapes span several tiles with ragged tails; the
full-size workloads are compared on every element (c3 prefill, c3 decode, c5) or on 16
(batch, head) pairs of every row (the long causal c4 cases)."""
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


def dense_mask(seed, Lq, Lk):
    rng = np.random.default_rng(seed)
    m = rng.standard_normal((Lq, Lk)).astype(np.float32)
    m[rng.random((Lq, Lk)) < 0.4] = -np.inf
    m[1] = -np.inf                       # a fully masked row
    m[2, :] = -np.inf
    m[2, Lk // 2:Lk // 2 + 3] = 1.5      # a row with three finite, non-zero entries
    return m


SMALL = []
for dtype, d in (("bf16", 128), ("bf16", 64), ("fp16", 128), ("fp16", 64), ("fp32", 64), ("fp32", 40)):
    for kind in ("none", "causal", "window", "dense", "topk"):
        SMALL.append((dtype, d, kind))


@pytest.mark.parametrize("dtype,d,kind", SMALL)
def test_small_ragged(dtype, d, kind):
    B, Hq, Hkv, Lq, Lk = 2, 4, 2, 77, 203
    p = synth.make_problem(f"small {dtype} d{d} {kind}", B, Hq, Hkv, Lq, Lk, d, dtype, kind, 100 + d,
                           window_left=37, keep_k=17, with_zero_hold=kind == "topk",
                           mask=dense_mask(7, Lq, Lk) if kind == "dense" else None)
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("Lq,Lk,kind", [(130, 50, "causal"), (1, 1000, "causal"), (3, 517, "window"),
                                         (64, 64, "topk"), (1, 1, "none"), (200, 129, "topk")])
def test_edge_shapes(dtype, Lq, Lk, kind):
    d = 128 if dtype == "bf16" else 64
    p = synth.make_problem(f"edge {dtype} Lq{Lq} Lk{Lk} {kind}", 1, 8, 1, Lq, Lk, d, dtype, kind, 200 + Lq,
                           window_left=5, keep_k=9, with_zero_hold=kind == "topk")
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


@pytest.mark.parametrize("name", ["c1", "c2", "c2b", "c2c", "c2w"])
def test_small_configs_full(name):
    p = synth.config(name)
    say(f"config {name}: {p.name}")
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=name)
    if name == "c2b":
        assert np.all(out == 0) and np.all(lse == -np.inf)
    if name == "c2c":   # one visible key per row: out = v[pos] rounded, lse = its logit
        v = p.f64("v")
        for i in range(p.Lq):
            np.testing.assert_allclose(out[:, :, i], np.repeat(v[:, :, 572 + i], p.Hq // p.Hkv, axis=1),
                                       rtol=0, atol=1e-2)


@pytest.mark.parametrize("Lq,Lk,path", [(16, 2900, 1), (3, 2900, 2), (130, 4100, 1), (16, 700, 1)])
def test_dense_mask_with_and_without_summary(Lq, Lk, path):
    """Dense masks over long key ranges build per-tile summary flags and skip the tiles
    the mask hides (mostly hidden here: a window of 200 keys, and a block of keys near
    the start visible to a few rows); short ranges visit every tile. Both against the
    oracle, on the prefill and decode paths."""
    import masked_flashattention_forward_amd as mfa
    m = synth.window_dense_mask(Lq, Lk, Lk - Lq, 200)
    m[: max(1, Lq // 3), 70:90] = 0.5
    p = synth.make_problem(f"dense summary Lq{Lq} Lk{Lk} path{path}", 2, 8, 2, Lq, Lk, 128, "bf16", "dense",
                           1500 + Lk + Lq, mask=m)
    pl = mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, "dense")
    assert pl["mask_summary"] == (Lk >= 2048), pl
    say(p.name)
    try:
        mfa.set_debug(force_path=path)
        out, lse = run_gpu(p, out_fill=float("nan"))
    finally:
        mfa.set_debug()
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


def test_c2_dense_equals_window_kind():
    """Two routes on the GPU: the dense window mask over 700 keys and the window kind
    over the first 576 keys give the same result."""
    a = run_gpu(synth.config("c2"))
    b = run_gpu(synth.config("c2w"))
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=2e-2)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-3)


def test_no_skip_switch_changes_nothing():
    import masked_flashattention_forward_amd as mfa
    for kind in ("causal", "window", "dense", "topk"):
        p = synth.make_problem(f"noskip {kind}", 1, 4, 1, 100, 700, 128, "bf16", kind, 300,
                               window_left=60, keep_k=30, with_zero_hold=kind == "topk",
                               mask=synth.window_dense_mask(100, 700, 500, 60) if kind == "dense" else None)
        say(p.name)
        a = run_gpu(p)
        try:
            mfa.set_debug(no_skip=True)
            b = run_gpu(p)
        finally:
            mfa.set_debug()
        # Skipping only drops keys that are -inf for every row of a tile, but it moves the
        # chunk boundaries, so the fp32 summation order changes and an output may round to
        # the neighbouring bf16 value (one ulp, 2^-7 relative). Top-k with skipping runs over
        # each block's kept-key list, so its tiles hold other keys and its running maxima
        # move at other tiles: P is rounded to bf16 against another reference, and each
        # weight may differ by 2^-8 relative between the routes, bounding the output
        # difference by 2^-8 * max|v|.
        np.testing.assert_array_equal(a[1] == -np.inf, b[1] == -np.inf)
        atol = 2.0**-8 * float(np.abs(p.f64("v")).max()) if kind == "topk" else 1e-3
        np.testing.assert_allclose(a[0], b[0], rtol=2.0**-7, atol=atol)
        fin = np.isfinite(a[1])
        np.testing.assert_allclose(a[1][fin], b[1][fin], rtol=0, atol=1e-4)


def test_runs_are_bitwise_deterministic():
    p = synth.make_problem("determinism", 2, 8, 2, 300, 900, 128, "bf16", "causal", 301)
    say(p.name)
    a = run_gpu(p)
    b = run_gpu(p)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("kind", ["causal", "window", "dense", "topk", "none"])
@pytest.mark.parametrize("splits", [1, 2, 3, 7])
@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("d", [128, 64])
def test_forced_split_kv_merge(kind, splits, path, d):
    """Split-KV with the LSE merge on the prefill kernel (path 1) and the decode kernel
    (path 2), including splits whose key range is empty or fully masked (window), against
    the oracle."""
    import masked_flashattention_forward_amd as mfa
    Lq, Lk = 5, 1111
    p = synth.make_problem(f"path{path} split{splits} d{d} {kind}", 2, 8, 2, Lq, Lk, d, "bf16", kind,
                           400 + splits, window_left=70, keep_k=50, with_zero_hold=kind == "topk",
                           mask=synth.window_dense_mask(Lq, Lk, 900, 100) if kind == "dense" else None)
    say(p.name)
    try:
        mfa.set_debug(force_path=path, force_splits=splits)
        out, lse = run_gpu(p, out_fill=float("nan"))
    finally:
        mfa.set_debug()
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_row_kernel_and_mfma_agree(dtype):
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem(f"paths {dtype}", 1, 4, 4, 150, 333, 64, dtype, "causal", 500)
    say(p.name)
    a = run_gpu(p)
    try:
        mfa.set_debug(force_path=0)
        b = run_gpu(p)
    finally:
        mfa.set_debug()
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=2e-2)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-3)


@pytest.mark.parametrize("G,Lq,Lk,path", [(96, 7, 300, "mfma_prefill"), (128, 5, 700, "mfma_prefill"),
                                          (256, 3, 200, "row")])
@pytest.mark.parametrize("kind", ["causal", "topk"])
def test_largest_head_groups(G, Lq, Lk, path, kind):
    """One KV head read by 96, 128 (the most a 128-row prefill block takes: one query
    position per block) and 256 query heads (more than a block holds: the row kernel)."""
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem(f"G{G} {kind} Lq{Lq} Lk{Lk}", 1, G, 1, Lq, Lk, 128, "bf16", kind, 1800 + G,
                           keep_k=50, with_zero_hold=kind == "topk")
    assert mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, kind, keep_k=p.keep_k)["path"] == path
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


@pytest.mark.parametrize("dtype,d,Lq,Lk,path", [("bf16", 128, 200, 700, "mfma_prefill"),
                                               ("fp16", 64, 300, 300, "mfma_prefill"),
                                               ("bf16", 128, 1, 3000, "splitkv_decode"), ("fp32", 64, 40, 90, "row")])
def test_zero_scale_weighs_visible_keys_equally(dtype, d, Lq, Lk, path):
    """scale = 0: every visible key gets the same weight, so each row's output is the mean
    of its visible V rows and its LSE is ln(number of visible keys) (causal: Lk - Lq + i + 1
    keys for row i). Checked against that closed form directly, not only the oracle."""
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem(f"zero scale {dtype} d{d} {Lq}x{Lk}", 2, 4, 2, Lq, Lk, d, dtype, "causal", 1900 + Lq,
                           scale=0.0)
    assert mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, "causal", dtype=synth.DTYPE_CODES[dtype])["path"] == path
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    v = p.f64("v")
    n_vis = Lk - Lq + np.arange(Lq) + 1
    mean_v = np.cumsum(v, axis=2)[:, :, Lk - Lq:, :] / n_vis[None, None, :, None]
    ref_o = np.repeat(mean_v, p.Hq // p.Hkv, axis=1)
    ref_l = np.broadcast_to(np.log(n_vis.astype(np.float64)), lse.shape)
    compare(p, out, lse, ref_o, ref_l, label=p.name)
    o2, l2 = run_oracle(p)
    np.testing.assert_allclose(o2, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, ref_l, rtol=0, atol=1e-12)


@pytest.mark.parametrize("G,Lq", [(4, 1), (8, 4), (32, 1), (1, 32), (6, 5)])
def test_decode_path_shapes(G, Lq):
    """Shapes the planner sends to the split-KV decode kernel (G * Lq <= 32)."""
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem(f"decode G{G} Lq{Lq}", 2, 2 * G, 2, Lq, 3000, 128, "fp16", "causal", 600 + G)
    assert mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, "causal", dtype=mfa.F16)["path"] == "splitkv_decode"
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lk,keep", [(1, 2, 2, 1024, 1024, 128), (2, 8, 2, 300, 1500, 200),
                                                   (1, 8, 2, 300, 200, 20)])
def test_topk_kept_key_lists(B, Hq, Hkv, Lq, Lk, keep):
    """Top-k attention over each query block's kept-key list (the gathered tiles): square,
    with past keys under GQA, and with more queries than keys (the first blocks' rows see
    no key, so their lists are empty), against the oracle."""
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem(f"topk lists {B}x{Hq}/{Hkv} {Lq}x{Lk} keep {keep}", B, Hq, Hkv, Lq, Lk, 128, "bf16",
                           "topk", 700 + keep, keep_k=keep, with_zero_hold=True)
    assert mfa.plan(B, Hq, Hkv, Lq, Lk, 128, "topk", keep_k=keep)["topk_list_cap"] > 0
    say(p.name)
    out, lse = run_gpu(p, out_fill=float("nan"))
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=p.name)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c3p", "c3d", "c5"])
def test_full_size_every_element(name):
    """The timed workloads at full size, in the launch configuration the benchmark uses
    (the plan depends on the shape only), compared element by element on every batch,
    head and row: this covers the workgroup remap over the XCDs, the heavy-first query
    block order, the split rule and the full kept-key lists, which only run at this size.
    The output starts filled with NaN, so a row no workgroup writes fails."""
    p = synth.config(name)
    say(f"config {name}: {p.name} (every element)")
    out, lse = run_gpu(p, out_fill=float("nan"))
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    ref_o, ref_l = run_oracle(p)
    compare(p, out, lse, ref_o, ref_l, label=f"{name} every element")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c4_d128_bf16", "c4_d64_bf16", "c4_d128_fp16", "c4_d64_fp16"])
def test_full_size_long_causal_16_heads(name):
    """The long causal workloads (64 (batch, head) pairs of 8192 x 8192) at full size:
    every output checked for NaN, and 16 seeded (batch, head) pairs, the first and last
    included, on every row against the oracle."""
    p = synth.config(name)
    say(f"config {name}: {p.name} (16 heads, every row)")
    out, lse = run_gpu(p, out_fill=float("nan"))
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    rng = np.random.default_rng(123)
    pairs = [(b, h) for b in range(p.B) for h in range(p.Hq)]
    pick = rng.choice(len(pairs), size=14, replace=False)
    heads = sorted({pairs[0], pairs[-1]} | {pairs[int(i)] for i in pick})
    while len(heads) < 16:
        heads = sorted(set(heads) | {pairs[int(rng.integers(len(pairs)))]})
    ref_o, ref_l = run_oracle(p, heads=heads)
    compare(p, out, lse, ref_o, ref_l, heads=heads, label=f"{name} 16 heads")
