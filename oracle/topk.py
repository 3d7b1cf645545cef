"""Dynamic top-k mask, plain definitions (fp64/int64, CPU).

TEST INFRASTRUCTURE: see the package docstring.

The flash-sparse-attention issue page ("Overview", "Current Status") builds
the dynamic mask from per-key ``zero_hold_states`` computed ahead of the
kernel, combining causal masking with a top-k selection sized by
``keep_window_size``; it never prints the formula. The reading used here
(stated once, used by every function below):

* selection is among the causally allowed keys of a query row (keys at or
  before the row's bottom-right-aligned position), or among all keys when
  ``causal`` is false;
* keys are ordered by zero_hold value, largest first, ties broken by the
  lower key index; -0.0 and +0.0 compare equal;
* the first ``keep_k`` keys of that order are kept, so a row with at most
  ``keep_k`` allowed keys keeps all of them;
* a kept key adds its zero_hold value to the scaled logit; every other key
  is -inf.
"""
from __future__ import annotations

import numpy as np

from .attention import query_positions

INT32_MAX = np.iinfo(np.int32).max


def _canon(zh_row: np.ndarray) -> np.ndarray:
    z = np.asarray(zh_row, dtype=np.float64).copy()
    z[z == 0.0] = 0.0        # fold -0.0 into +0.0
    return z


def topk_kept_ref(zh_row: np.ndarray, Lq: int, keep_k: int, causal: bool = True, rows=None) -> np.ndarray:
    """bool [Lq, Lk] (or [len(rows), Lk]): the kept set of each query row, by the definition.

    For each row: list the allowed keys, stable-sort them by descending
    zero_hold (a stable sort keeps lower indices first among ties), keep the
    first ``keep_k``. Pinned by brute force and by the hand-enumerated
    minimal example of the flash-sparse-attention page ("Next Steps", item 4).
    """
    z = _canon(zh_row)
    Lk = z.shape[0]
    pos = query_positions(Lq, Lk)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    kept = np.zeros((rows.size, Lk), dtype=bool)
    for r, i in enumerate(rows):
        n_allowed = (min(Lk, pos[i] + 1) if pos[i] >= 0 else 0) if causal else Lk
        if n_allowed <= 0:
            continue
        cand = np.arange(n_allowed)
        order = cand[np.argsort(-z[:n_allowed], kind="stable")]
        kept[r, order[:keep_k]] = True
    return kept


def topk_rank_ref(zh_row: np.ndarray) -> np.ndarray:
    """int64 [Lk]: each key's place in the total order (zero_hold descending,
    key index ascending). Unique for NaN-free input, so GPU ranks must match
    bit for bit."""
    z = _canon(zh_row)
    Lk = z.shape[0]
    order = np.lexsort((np.arange(Lk), -z))
    rank = np.empty(Lk, dtype=np.int64)
    rank[order] = np.arange(Lk)
    return rank


def topk_tau_ref(rank: np.ndarray, Lq: int, keep_k: int, causal: bool = True) -> np.ndarray:
    """int64 [Lq]: per-row rank threshold.

    A row keeps key j iff j is allowed and ``rank[j] <= tau``. When the row
    has more than ``keep_k`` allowed keys, tau is the ``keep_k``-th smallest
    rank among them; otherwise every allowed key is kept and tau is INT32_MAX.
    """
    rank = np.asarray(rank)
    Lk = rank.shape[0]
    pos = query_positions(Lq, Lk)
    tau = np.full(Lq, INT32_MAX, dtype=np.int64)
    for i in range(Lq):
        n_allowed = (min(Lk, pos[i] + 1) if pos[i] >= 0 else 0) if causal else Lk
        if n_allowed > keep_k:
            tau[i] = np.partition(rank[:n_allowed], keep_k - 1)[keep_k - 1]
    return tau


def kept_from_rank_tau(rank: np.ndarray, tau: np.ndarray, Lq: int, causal: bool = True) -> np.ndarray:
    """bool [Lq, Lk] rebuilt from (rank, tau)."""
    rank = np.asarray(rank)
    Lk = rank.shape[0]
    pos = query_positions(Lq, Lk)
    ok = rank[None, :] <= np.asarray(tau)[:, None]
    if causal:
        ok &= np.arange(Lk)[None, :] <= pos[:, None]
    return ok


def pack_keep_bits(kept: np.ndarray) -> np.ndarray:
    """uint32 [..., ceil(Lk/32)]: bit (j mod 32) of word (j div 32) is key j."""
    kept = np.asarray(kept, dtype=bool)
    Lk = kept.shape[-1]
    nw = (Lk + 31) // 32
    pad = np.zeros(kept.shape[:-1] + (nw * 32,), dtype=np.uint64)
    pad[..., :Lk] = kept
    pad = pad.reshape(kept.shape[:-1] + (nw, 32))
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (pad * weights).sum(axis=-1).astype(np.uint32)
