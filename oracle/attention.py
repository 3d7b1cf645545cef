"""Masked softmax attention forward, plain fp64 definitions (CPU).

TEST INFRASTRUCTURE: see the package docstring.

Readings of the pages used below (each also listed in the design notes):

* Query row ``i`` of ``Lq`` rows against ``Lk`` keys sits at absolute
  position ``p_i = Lk - Lq + i`` (bottom-right alignment). This is the only
  reading under which causal attention with past keys equals the padded
  computation that the FastChat page ("Enable use_cache support with
  Flash-Attention") calls the old, slower workaround.
* Causal: key j is visible iff ``j <= p_i``. Window ``W``: iff
  ``p_i - W <= j <= p_i`` (inclusive; the ExecuTorch page's example decodes
  position 575 against keys 515..575).
* Dense: an fp32 ``[Lq, Lk]`` additive mask, the same for every batch and
  head, added to the scaled logits before the softmax (ExecuTorch page,
  "Summary"; flash-sparse-attention page, "Next Steps" item 1). Only -inf
  masks a key.
* Top-k: see ``topk.py``.
* A row whose every logit is -inf returns output 0 and LSE = -inf.
* LSE is the natural-log log-sum-exp of the masked, biased, scaled logits.
* GQA/MQA: query head h reads KV head ``h // (Hq // Hkv)`` (InfiniTrain
  page, "Framework and autograd": MHA when Hq == Hkv, GQA/MQA when
  Hq % Hkv == 0, an error otherwise).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def query_positions(Lq: int, Lk: int) -> np.ndarray:
    """Absolute key position of each query row (bottom-right alignment)."""
    return np.arange(Lq, dtype=np.int64) + (Lk - Lq)


def mask_matrix(kind: str, Lq: int, Lk: int, *, window_left: int = 0, dense=None,
                zh_row=None, keep_k: int = 0, rows=None) -> np.ndarray:
    """fp64 additive mask ``A[i, j]`` for the requested rows (all rows by default)."""
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    pos = query_positions(Lq, Lk)[rows][:, None]
    j = np.arange(Lk)[None, :]
    if kind == "none":
        return np.zeros((rows.size, Lk))
    if kind == "causal":
        return np.where(j <= pos, 0.0, NEG_INF)
    if kind == "window":
        return np.where((j <= pos) & (j >= pos - window_left), 0.0, NEG_INF)
    if kind == "dense":
        return np.asarray(dense, dtype=np.float64)[rows]
    if kind == "topk":
        from .topk import topk_kept_ref
        kept = topk_kept_ref(zh_row, Lq, keep_k, causal=True, rows=rows)
        return np.where(kept, np.asarray(zh_row, dtype=np.float64)[None, :], NEG_INF)
    raise ValueError(kind)


def attention_rows_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                       A: np.ndarray):
    """One head: q ``[n, d]``, k/v ``[Lk, d]``, additive mask A ``[n, Lk]``.

    Returns (out ``[n, d]``, lse ``[n]``) in fp64, computed by materialising
    ``Z = scale * q k^T + A`` and its softmax.
    """
    Z = scale * (q @ k.T) + A
    M = Z.max(axis=1)
    dead = M == NEG_INF
    M0 = np.where(dead, 0.0, M)
    W = np.exp(Z - M0[:, None])          # exp(-inf) = 0 for masked keys
    l = W.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = (W @ v) / l[:, None]
        lse = M0 + np.log(l)
    out[dead] = 0.0
    lse[dead] = NEG_INF
    return out, lse


def attention_ref(q, k, v, scale, kind, *, window_left=0, mask=None, zero_hold=None,
                  keep_k=0, rows=None, heads=None):
    """Full multi-head forward.

    q ``[B,Hq,Lq,d]``, k/v ``[B,Hkv,Lk,d]`` (fp64 values of the stored inputs),
    mask ``[Lq,Lk]``, zero_hold ``[B,Hkv,Lk]``.
    ``rows`` restricts the query rows computed (all by default); ``heads`` is
    an optional list of (b, h) pairs (all by default). Unrequested entries of
    the returned arrays are NaN.
    """
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    rows_idx = np.arange(Lq) if rows is None else np.asarray(rows)
    out = np.full((B, Hq, Lq, d), np.nan)
    lse = np.full((B, Hq, Lq), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    cache = {}
    for b, h in heads:
        g = h // G
        key = (b, g) if kind == "topk" else None
        if key not in cache:
            zh = None if zero_hold is None else zero_hold[b, g]
            cache[key] = mask_matrix(kind, Lq, Lk, window_left=window_left, dense=mask,
                                     zh_row=zh, keep_k=keep_k, rows=rows_idx)
        o, s = attention_rows_ref(q[b, h, rows_idx], k[b, g], v[b, g], scale, cache[key])
        out[b, h, rows_idx] = o
        lse[b, h, rows_idx] = s
    return out, lse


def attention_chunked_ref(q, k, v, scale, A, chunk: int, guard: bool = True):
    """Second route for one head: online softmax over key chunks of ``chunk``.

    Running state per row: max ``m``, sum ``l``, unnormalised output ``acc``.
    For each chunk: ``m_new = max(m, max z)``; the guard replaces an all -inf
    ``m_new`` by 0 before it is subtracted, so a chunk that is entirely -inf
    rescales by ``exp(-inf) = 0`` instead of ``exp(-inf - -inf) = NaN`` (the
    failure the ExecuTorch page, "Summary", describes for a 512-key chunk).
    With ``guard=False`` the unguarded update is used, which yields NaN there.
    """
    n, Lk = A.shape
    m = np.full(n, NEG_INF)
    l = np.zeros(n)
    acc = np.zeros((n, v.shape[1]))
    for j0 in range(0, Lk, chunk):
        z = scale * (q @ k[j0:j0 + chunk].T) + A[:, j0:j0 + chunk]
        m_new = np.maximum(m, z.max(axis=1))
        ref = np.where(m_new == NEG_INF, 0.0, m_new) if guard else m_new
        with np.errstate(invalid="ignore"):
            alpha = np.exp(m - ref)
            p = np.exp(z - ref[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j0 + chunk]
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        out = acc / l[:, None]
        ref = np.where(m == NEG_INF, 0.0, m) if guard else m
        lse = ref + np.log(l)
    if guard:
        dead = l == 0.0
        out[dead] = 0.0
        lse[dead] = NEG_INF
    return out, lse


def lse_merge_ref(outs: np.ndarray, lses: np.ndarray):
    """Combine partial results over disjoint key ranges.

    ``outs`` ``[S, ..., d]`` are per-part normalised outputs, ``lses`` ``[S, ...]``
    their log-sum-exps. ``lse = log sum_s exp(lse_s)`` (all parts -inf gives
    -inf and output 0) and ``out = sum_s exp(lse_s - lse) * out_s``.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    dead = M == NEG_INF
    M0 = np.where(dead, 0.0, M)
    w = np.exp(lses - M0)
    tot = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = M0 + np.log(tot)
        out = (w[..., None] * np.nan_to_num(outs)).sum(axis=0) / tot[..., None]
    lse = np.where(dead, NEG_INF, lse)
    out[dead] = 0.0
    return out, lse
