"""The work counts bench.py divides by, checked on small problems against brute force over
the oracle's mask matrices (no GPU): visible (row, key) pairs per mask kind, and the
algorithmic bytes' count of distinct visible keys."""
import numpy as np
import pytest

import bench
import synth
from oracle import mask_matrix


def brute_pairs(p):
    total = 0
    for b in range(p.B):
        for g in range(p.Hkv):
            A = mask_matrix(p.mask_kind, p.Lq, p.Lk, window_left=p.window_left,
                            dense=None if p.mask is None else p.mask.astype(np.float64),
                            zh_row=None if p.zero_hold is None else p.zero_hold[b, g].astype(np.float64),
                            keep_k=p.keep_k)
            total += int(np.isfinite(A).sum()) * (p.Hq // p.Hkv)
    return total


@pytest.mark.parametrize("kind", ["none", "causal", "window", "dense", "topk"])
@pytest.mark.parametrize("Lq,Lk", [(7, 23), (23, 7), (16, 16), (1, 40)])
def test_visible_pairs_match_brute_force(kind, Lq, Lk):
    rng = np.random.default_rng(Lq * 100 + Lk)
    mask = None
    if kind == "dense":
        mask = rng.standard_normal((Lq, Lk)).astype(np.float32)
        mask[rng.random((Lq, Lk)) < 0.5] = -np.inf
    p = synth.make_problem("count", 2, 4, 2, Lq, Lk, 8, "fp32", kind, 3, window_left=5, keep_k=4,
                           with_zero_hold=kind == "topk", mask=mask)
    assert bench.visible_pairs(p) == brute_pairs(p)


@pytest.mark.parametrize("Lq,Lk", [(7, 23), (23, 7), (16, 16)])
def test_causal_pairs_and_headline_flops(Lq, Lk):
    p = synth.make_problem("count", 1, 2, 1, Lq, Lk, 8, "fp32", "causal", 3)
    assert bench.causal_pairs(p) == brute_pairs(p)


def test_headline_flop_count():
    """c3 prefill: 257.73 GFLOP per call (4 d flop per visible pair), the figure the
    roofline divides by."""
    Lq, Lk, heads, d = 512, 4096, 8 * 32, 128
    pairs = sum(min(Lk, Lk - Lq + i + 1) for i in range(Lq)) * heads
    assert 4 * d * pairs == 257731592192


@pytest.mark.parametrize("kind", ["causal", "window", "dense", "none"])
def test_algorithmic_bytes_count_distinct_visible_keys(kind):
    rng = np.random.default_rng(9)
    Lq, Lk = 9, 30
    mask = None
    if kind == "dense":
        mask = np.full((Lq, Lk), -np.inf, dtype=np.float32)
        mask[:, 3:11] = 0.0
    p = synth.make_problem("bytes", 2, 4, 2, Lq, Lk, 8, "bf16", kind, 4, window_left=4, mask=mask)
    A = mask_matrix(kind, Lq, Lk, window_left=4, dense=None if mask is None else mask.astype(np.float64))
    keys = int(np.isfinite(A).any(axis=0).sum())
    es = 2
    expect = 2 * p.B * p.Hq * Lq * 8 * es + p.B * p.Hq * Lq * 4 + 2 * p.B * p.Hkv * keys * 8 * es
    if kind == "dense":
        expect += mask.nbytes
    assert bench.algorithmic_bytes(p) == expect


def test_configs_subset_option():
    """--configs names entries of the per-configuration list; an unknown name stops the run
    before anything is measured (exit status 2, the known names listed)."""
    import subprocess
    import sys
    names = bench.config_entry_names()
    assert len(names) == len(set(names))
    assert {"c3d", "c5", "serve", "c4_d128_bf16_bwd", "c3p_bwd"} <= set(names)
    r = subprocess.run([sys.executable, "bench.py", "--configs", "c3d,not_a_config"], capture_output=True, text=True,
                       cwd=bench.__file__.rsplit("/", 1)[0], timeout=120)
    assert r.returncode == 2 and "not_a_config" in r.stderr and "c4_d128_bf16_bwd" in r.stderr
