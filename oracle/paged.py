"""Attention over a batch of sequences of different lengths whose keys and values sit
in a paged cache (or packed back to back), plain fp64 definitions (CPU).

TEST INFRASTRUCTURE: see the package docstring.

The interface follows the vLLM pull request #11277 page (the unified varlen call its
reviewers ask to align with): queries of all sequences packed token-major with
``cu_seqlens_q`` offsets, key counts given by the differences of ``cu_seqlens_k``, and
a block table mapping a sequence's logical cache pages to physical pages. The same page
describes the alternative of passing the cached keys and the new tokens' own keys
("cached KV and active KV") separately instead of writing the new ones into the cache
first; ``k_new``/``v_new`` select that form.

Readings (the page names the arguments only; everything below is the plainest reading):

* Paged layout ``[num_pages, page_size, Hkv, d]``: key ``j`` of sequence ``s`` is slot
  ``j % page_size`` of page ``block_table[s, j // page_size]``.
* Without a block table K/V are packed ``[total_k, Hkv, d]`` and sequence ``s`` owns rows
  ``cu_seqlens_k[s] .. cu_seqlens_k[s+1] - 1``.
* Query ``i`` of a sequence with ``Lq`` queries and ``Lk`` keys sits at position
  ``Lk - Lq + i`` (bottom-right, as for the single-batch forward).
* With ``k_new``/``v_new`` ``[total_q, Hkv, d]`` the last ``Lq`` keys of a sequence are
  its own new tokens (row ``cu_seqlens_q[s] + i`` is key ``Lk - Lq + i``) and the cache
  holds the first ``Lk - Lq``. A sequence with fewer keys than queries has no such
  split; its rows are returned fully masked (output 0, LSE -inf).
* LSE is returned token-major, ``[total_q, Hq]``.
* The score modifiers of the same call (``alibi_slopes``, ``softcap``) apply as in
  ``general.py``, on each sequence's own positions: the ALiBi distance of key ``j`` from
  query ``i`` of sequence ``s`` is ``|Lk_s - Lq_s + i - j|``.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_ref
from .general import general_attention_ref


def gather_sequence_kv(cache: np.ndarray, table_row, page_size: int, n: int) -> np.ndarray:
    """Keys (or values) ``0..n-1`` of one sequence from a paged cache: ``[Hkv, n, d]``."""
    j = np.arange(n)
    pages = np.asarray(table_row, dtype=np.int64)[j // page_size]
    return np.ascontiguousarray(cache[pages, j % page_size].transpose(1, 0, 2))


def _sequence_kv(cache, block_table, page_size, cu_k, s, n):
    """The first ``n`` keys (values) of sequence ``s``, paged or packed: ``[Hkv, n, d]``."""
    if block_table is None:
        k0 = int(cu_k[s])
        return np.ascontiguousarray(np.asarray(cache[k0:k0 + n], dtype=np.float64).transpose(1, 0, 2))
    return gather_sequence_kv(np.asarray(cache, dtype=np.float64), block_table[s], page_size, n)


def paged_attention_ref(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_table, page_size, scale, kind,
                        *, window_left=0, k_new=None, v_new=None, alibi_slopes=None, softcap=0.0):
    """q ``[total_q, Hq, d]``; returns out ``[total_q, Hq, d]`` and lse ``[total_q, Hq]``.

    ``block_table`` ``[num_seqs, max_pages]`` (or None for packed K/V); ``kind`` is one of
    the key-position masks ("none", "causal", "window"); ``alibi_slopes`` ``[Hq]`` or None.
    """
    mods = alibi_slopes is not None or softcap > 0.0
    q = np.asarray(q, dtype=np.float64)
    total_q, Hq, d = q.shape
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    Hkv = k_cache.shape[-2]
    out = np.zeros((total_q, Hq, d))
    lse = np.full((total_q, Hq), -np.inf)
    for s in range(cu_q.size - 1):
        q0, q1 = int(cu_q[s]), int(cu_q[s + 1])
        Lq, Lk = q1 - q0, int(cu_k[s + 1] - cu_k[s])
        if Lq == 0:
            continue
        if k_new is None:
            K = _sequence_kv(k_cache, block_table, page_size, cu_k, s, Lk)
            V = _sequence_kv(v_cache, block_table, page_size, cu_k, s, Lk)
        else:
            ctx = Lk - Lq
            if ctx < 0:
                continue  # no cached/new split: rows stay fully masked
            K = np.concatenate([_sequence_kv(k_cache, block_table, page_size, cu_k, s, ctx),
                                np.asarray(k_new[q0:q1], dtype=np.float64).transpose(1, 0, 2)], axis=1)
            V = np.concatenate([_sequence_kv(v_cache, block_table, page_size, cu_k, s, ctx),
                                np.asarray(v_new[q0:q1], dtype=np.float64).transpose(1, 0, 2)], axis=1)
        if Lk == 0:
            continue  # no key at all: every row is fully masked
        Q = q[q0:q1].transpose(1, 0, 2)[None]
        if mods:
            o, l = general_attention_ref(Q, K.reshape(1, Hkv, Lk, d), V.reshape(1, Hkv, Lk, d), scale, kind,
                                         window_left=window_left, alibi_slopes=alibi_slopes, softcap=softcap)
        else:
            o, l = attention_ref(Q, K.reshape(1, Hkv, Lk, d), V.reshape(1, Hkv, Lk, d), scale, kind,
                                 window_left=window_left)
        out[q0:q1] = o[0].transpose(1, 0, 2)
        lse[q0:q1] = l[0].T
    return out, lse
