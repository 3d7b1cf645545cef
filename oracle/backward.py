"""Gradients of the masked attention forward, plain fp64 definitions (CPU).

TEST INFRASTRUCTURE: see the package docstring.

The InfiniTrain pull request #193 page integrates forward and backward kernels for the
same attention ("main changes": fwd/bwd for FP16 and BF16, head dims 64 and 128; the
autograd function saves what the backward needs, "Framework and autograd"). The pages
give no formula; the backward of softmax attention is the plain chain rule of the
forward in ``attention.py``, written out here without any blocking:

  Z = scale * q k^T + A          (A: the additive mask; no gradient flows into it)
  P = softmax(Z) by rows          (a row with every logit -inf has P = 0, out = 0)
  O = P v
  dv = P^T dO
  dP = dO v^T
  dZ = P * (dP - rowsum(dP * P))  (the softmax Jacobian; rowsum(dP * P) = rowsum(dO * O))
  dq = scale * dZ k
  dk = scale * dZ^T q

With GQA a KV head's dk and dv are the sums over the query heads that read it. The top-k
mask enters only through A (its zero_hold values are inputs, not trained).
"""
from __future__ import annotations

import numpy as np

from .attention import NEG_INF, mask_matrix


def softmax_backward_terms(q, k, v, dout, scale, A):
    """One head's intermediate quantities of the definition above: P ``[n, Lk]`` and
    dZ ``[n, Lk]`` (fp64)."""
    Z = scale * (q @ k.T) + A
    M = Z.max(axis=1)
    dead = M == NEG_INF
    M0 = np.where(dead, 0.0, M)
    W = np.exp(Z - M0[:, None])
    l = W.sum(axis=1)
    P = np.zeros_like(W)
    P[~dead] = W[~dead] / l[~dead, None]
    dP = dout @ v.T
    dZ = P * (dP - (dP * P).sum(axis=1, keepdims=True))
    return P, dZ


def attention_backward_rows_ref(q, k, v, dout, scale, A):
    """One head: q ``[n, d]``, k/v ``[Lk, d]``, dout ``[n, d]``, mask A ``[n, Lk]``.
    Returns (dq ``[n, d]``, dk ``[Lk, d]``, dv ``[Lk, d]``) in fp64."""
    P, dZ = softmax_backward_terms(q, k, v, dout, scale, A)
    dv = P.T @ dout
    dq = scale * (dZ @ k)
    dk = scale * (dZ.T @ q)
    return dq, dk, dv


def attention_backward_ref(q, k, v, dout, scale, kind, *, window_left=0, mask=None, zero_hold=None, keep_k=0):
    """Full backward. q/dout ``[B,Hq,Lq,d]``, k/v ``[B,Hkv,Lk,d]`` (fp64 values of the stored
    inputs), mask ``[Lq,Lk]``, zero_hold ``[B,Hkv,Lk]``. Returns (dq, dk, dv) with the
    shapes of q, k and v."""
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            A = mask_matrix(kind, Lq, Lk, window_left=window_left, dense=mask,
                            zh_row=None if zero_hold is None else zero_hold[b, g], keep_k=keep_k)
            for h in range(g * G, (g + 1) * G):
                a, bk, bv = attention_backward_rows_ref(q[b, h], k[b, g], v[b, g], dout[b, h], scale, A)
                dq[b, h] = a
                dk[b, g] += bk
                dv[b, g] += bv
    return dq, dk, dv
