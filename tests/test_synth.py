"""The seeded input generator: determinism and the storage rounding."""
import numpy as np
import torch

import synth


def test_draws_are_deterministic_and_ordered():
    a = synth.make_problem("t", 1, 2, 1, 5, 9, 8, "bf16", "causal", 7, with_zero_hold=True)
    b = synth.make_problem("t", 1, 2, 1, 5, 9, 8, "bf16", "causal", 7, with_zero_hold=True)
    assert synth.sha256(a.q, a.k, a.v, a.zero_hold) == synth.sha256(b.q, b.k, b.v, b.zero_hold)
    rng = np.random.default_rng(7)
    q32 = rng.standard_normal((1, 2, 5, 8), dtype=np.float32)
    np.testing.assert_array_equal(a.f64("q"), torch.from_numpy(q32).to(torch.bfloat16).double().numpy())


def test_bf16_rounding_is_nearest_even_like_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000, dtype=np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0,
                                  np.inf, -np.inf, 3.4e38], dtype=np.float32)])
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1
    assert synth.bf16_bits_to_f64(bits[100000:100001])[0] == 1.0
    assert synth.bf16_bits_to_f64(bits[100001:100002])[0] == 1.0 + 2 ** -6


def test_fp16_storage_roundtrip():
    p = synth.make_problem("t", 1, 1, 1, 4, 4, 8, "fp16", "none", 3)
    assert p.q.dtype == np.float16
    np.testing.assert_array_equal(p.f64("q"), p.q.astype(np.float64))


def test_config_shapes():
    p = synth.config("c2w")
    c2 = synth.make_problem("x", 4, 32, 8, 16, 700, 128, "bf16", "dense", 2)
    assert p.k.shape == (4, 8, 576, 128)
    np.testing.assert_array_equal(p.k, c2.k[:, :, :576])
    np.testing.assert_array_equal(p.q, c2.q)
    m = synth.window_dense_mask(16, 700, 560, 60)
    assert np.isfinite(m[15]).sum() == 61 and np.isfinite(m[15, 515:576]).all()


def test_paged_problem_pages_are_disjoint_and_cover_the_cache():
    p = synth.paged_config("v1")
    assert p.total_q == sum([1, 37, 1, 130, 0, 5, 3]) and p.num_seqs == 7
    used = []
    for s in range(p.num_seqs):
        n = (int(p.k_lens[s]) + p.page_size - 1) // p.page_size
        used.extend(p.block_table[s, :n].tolist())
    assert len(used) == len(set(used))
    assert p.kv_rows == len(used) + 2          # two spare pages nobody uses
    assert all(0 <= x < p.kv_rows for x in used)
    a = synth.paged_config("v1")
    np.testing.assert_array_equal(a.k, p.k)
    np.testing.assert_array_equal(a.block_table, p.block_table)


def test_two_source_problem_caches_only_the_context():
    p = synth.make_paged_problem("t", [3, 1], [10, 4], 4, 2, 8, "bf16", "causal", 5, page_size=4,
                                 two_source=True, spare_pages=0)
    assert p.k_new.shape == (4, 2, 8) and p.k.shape == (2 + 1, 4, 2, 8)   # ceil(7/4) + ceil(3/4) pages


def test_serving_lengths_mix():
    q, k = synth.serving_lengths(62, 4, 512, (1024, 4096), 60, (1024, 16384))
    assert (q[:4] == 512).all() and (q[4:] == 1).all()
    assert (k[:4] >= 1024 + 512).all() and (k[4:] >= 1024).all() and (k[4:] <= 16385).all()
