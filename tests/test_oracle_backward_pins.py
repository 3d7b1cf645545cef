"""Pins for oracle/backward.py, checked against facts fixed outside that module: central
finite differences of the forward oracle (no use of the analytic formula), torch autograd
through its CPU fp64 scaled-dot-product attention (a library routine), GQA as the sum over
repeated heads, and fully masked rows. No GPU is used here."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_ref, mask_matrix
from oracle.backward import attention_backward_ref


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def loss(q, k, v, w, scale, kind, **kw):
    """L = sum(out * w): its gradient with respect to out is w."""
    out, _ = attention_ref(q, k, v, scale, kind, **kw)
    return float((out * w).sum())


def finite_difference(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("kind", ["none", "causal", "window", "dense", "topk"])
def test_gradients_match_central_differences(kind):
    B, Hq, Hkv, Lq, Lk, d = 1, 2, 1, 5, 7, 3
    q, k, v, w = rnd(1, B, Hq, Lq, d), rnd(2, B, Hkv, Lk, d), rnd(3, B, Hkv, Lk, d), rnd(4, B, Hq, Lq, d)
    kw = dict(window_left=2)
    if kind == "dense":
        m = rnd(5, Lq, Lk)
        m[m < -0.8] = -np.inf
        kw["mask"] = m
    if kind == "topk":
        kw.update(zero_hold=rnd(6, B, Hkv, Lk), keep_k=3)
    dq, dk, dv = attention_backward_ref(q, k, v, w, 0.7, kind, **kw)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = finite_difference(lambda: loss(q, k, v, w, 0.7, kind, **kw), x)
        np.testing.assert_allclose(g, fd, rtol=0, atol=1e-7)


@pytest.mark.parametrize("kind", ["none", "causal", "dense"])
def test_gradients_match_torch_autograd(kind):
    B, Hq, Hkv, Lq, Lk, d = 2, 4, 2, 9, 13, 8
    q, k, v, w = rnd(10, B, Hq, Lq, d), rnd(11, B, Hkv, Lk, d), rnd(12, B, Hkv, Lk, d), rnd(13, B, Hq, Lq, d)
    mask = None
    if kind == "dense":
        mask = rnd(14, Lq, Lk)
        mask[mask < -1.0] = -np.inf
    A = mask_matrix(kind, Lq, Lk, dense=mask)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(A), scale=0.4, enable_gqa=True)
    (o * torch.from_numpy(w)).sum().backward()
    dq, dk, dv = attention_backward_ref(q, k, v, w, 0.4, kind, mask=mask)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_gqa_gradients_are_sums_over_the_sharing_heads():
    B, Hq, Hkv, Lq, Lk, d = 1, 4, 2, 6, 10, 4
    q, k, v, w = rnd(20, B, Hq, Lq, d), rnd(21, B, Hkv, Lk, d), rnd(22, B, Hkv, Lk, d), rnd(23, B, Hq, Lq, d)
    dq, dk, dv = attention_backward_ref(q, k, v, w, 0.5, "causal")
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = attention_backward_ref(q, kr, vr, w, 0.5, "causal")
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, 2, Lk, d).sum(axis=2), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, 2, Lk, d).sum(axis=2), rtol=0, atol=1e-14)


def test_fully_masked_rows_give_no_gradient():
    B, H, Lq, Lk, d = 1, 1, 4, 6, 3
    q, k, v, w = rnd(30, B, H, Lq, d), rnd(31, B, H, Lk, d), rnd(32, B, H, Lk, d), rnd(33, B, H, Lq, d)
    m = rnd(34, Lq, Lk)
    m[2] = -np.inf
    dq, dk, dv = attention_backward_ref(q, k, v, w, 0.9, "dense", mask=m)
    assert np.all(dq[0, 0, 2] == 0.0)
    w2 = w.copy()
    w2[0, 0, 2] = 123.0   # the dead row's output gradient changes nothing
    dq2, dk2, dv2 = attention_backward_ref(q, k, v, w2, 0.9, "dense", mask=m)
    np.testing.assert_array_equal(dk2, dk)
    np.testing.assert_array_equal(dv2, dv)
