"""Masked attention forward with the general score modifiers, plain fp64 definitions (CPU).

TEST INFRASTRUCTURE: see the package docstring.

This extends ``attention.py`` with what the pages name but the five workloads do not
use: the score modifiers of the vLLM pull request #11277 page's varlen call
(``alibi_slopes`` and ``softcap``, listed in its "API alignment" request; the
InfiniTrain pull request #193 page lists both among its declared gaps, "TODO"), a dense
mask that differs per batch and head (the vLLM page's backend passes a precomputed mask
per layer, its reply point 3), and the two top-k variants the flash-sparse-attention
issue #11 page mentions (the non-causal selection its mask tests cover, "Current
Status"; a top-k mask on top of another additive mask).

Readings (the pages name these arguments without defining them; each is the plainest
reading, the convention of the varlen API the vLLM page quotes):

* Order: ``t = scale * q k^T``; softcap, when ``softcap > 0``, replaces ``t`` by
  ``softcap * tanh(t / softcap)``; ALiBi adds ``-slope_h * |p_i - j|`` (``p_i`` the
  bottom-right position of query row i, ``slope_h`` the slope of query head h); then the
  mask of the kind is added; then the guarded softmax of ``attention.py``.
* Dense mask: any array that broadcasts to ``[B, Hq, Lq, Lk]`` (numpy broadcasting, so a
  size-1 dimension is shared: ``[Lq, Lk]`` is the single mask of ``attention.py``).
* Top-k: the kept set is chosen from zero_hold alone (``topk.py``), causal or over all
  keys; a kept key adds its zero_hold value and, when a dense mask is given with the
  top-k kind, that mask's value too; every other key is -inf.
"""
from __future__ import annotations

import numpy as np

from .attention import NEG_INF, attention_rows_ref, query_positions
from .topk import topk_kept_ref


def general_scores(q, k, scale, pos, *, softcap=0.0, alibi_slope=0.0):
    """fp64 logits of one head before the mask: q ``[n, d]``, k ``[Lk, d]``, ``pos`` the
    absolute position of each of the n query rows."""
    t = scale * (q @ k.T)
    if softcap > 0.0:
        t = softcap * np.tanh(t / softcap)
    if alibi_slope != 0.0:
        j = np.arange(k.shape[0])[None, :]
        t = t - alibi_slope * np.abs(np.asarray(pos)[:, None] - j)
    return t


def general_mask(kind, Lq, Lk, *, window_left=0, dense2d=None, zh_row=None, keep_k=0, topk_causal=True):
    """fp64 additive mask ``[Lq, Lk]`` of one (b, h): the position masks, a dense slice, or
    top-k (optionally with a dense slice added to the kept keys)."""
    pos = query_positions(Lq, Lk)[:, None]
    j = np.arange(Lk)[None, :]
    if kind == "none":
        return np.zeros((Lq, Lk))
    if kind == "causal":
        return np.where(j <= pos, 0.0, NEG_INF)
    if kind == "window":
        return np.where((j <= pos) & (j >= pos - window_left), 0.0, NEG_INF)
    if kind == "dense":
        return np.asarray(dense2d, dtype=np.float64)
    if kind == "topk":
        kept = topk_kept_ref(zh_row, Lq, keep_k, causal=topk_causal)
        add = np.asarray(zh_row, dtype=np.float64)[None, :]
        if dense2d is not None:
            add = add + np.asarray(dense2d, dtype=np.float64)
        with np.errstate(invalid="ignore"):
            return np.where(kept, add, NEG_INF)
    raise ValueError(kind)


def general_attention_ref(q, k, v, scale, kind, *, window_left=0, mask=None, zero_hold=None, keep_k=0,
                          topk_causal=True, alibi_slopes=None, softcap=0.0, heads=None):
    """Full forward with the modifiers above.

    q ``[B,Hq,Lq,d]``, k/v ``[B,Hkv,Lk,d]`` (fp64 values of the stored inputs); ``mask``
    broadcastable to ``[B,Hq,Lq,Lk]``; ``zero_hold`` ``[B,Hkv,Lk]``; ``alibi_slopes``
    ``[Hq]`` or None. ``heads`` optionally restricts the (b, h) pairs computed (the other
    entries of the result are NaN). Returns (out ``[B,Hq,Lq,d]``, lse ``[B,Hq,Lq]``).
    """
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    full = None if mask is None else np.broadcast_to(np.asarray(mask, dtype=np.float64), (B, Hq, Lq, Lk))
    pos = query_positions(Lq, Lk)
    out = np.full((B, Hq, Lq, d), np.nan)
    lse = np.full((B, Hq, Lq), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in heads:
        g = h // G
        A = general_mask(kind, Lq, Lk, window_left=window_left, dense2d=None if full is None else full[b, h],
                         zh_row=None if zero_hold is None else zero_hold[b, g], keep_k=keep_k,
                         topk_causal=topk_causal)
        slope = 0.0 if alibi_slopes is None else float(alibi_slopes[h])
        t = general_scores(q[b, h], k[b, g], scale, pos, softcap=softcap, alibi_slope=slope)
        # attention_rows_ref forms scale * q k^T + A; pass the finished logits through A
        # with unit q and zero k instead of re-implementing the softmax
        o, s = attention_rows_ref(np.zeros((Lq, 1)), np.zeros((Lk, 1)), v[b, g], 1.0, t + A)
        out[b, h] = o
        lse[b, h] = s
    return out, lse
