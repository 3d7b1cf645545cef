"""Seeded synthetic inputs for the masked attention forward.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic: both the fp64 oracle and the HIP
path receive exactly the arrays built here.

Recipe (shared by tests and the benchmark):
  * generator: numpy ``default_rng(seed)`` (PCG64), ``standard_normal(...,
    dtype=float32)``, drawn in the order q, k, v, then zero_hold_states;
  * storage cast: round-to-nearest-even from fp32 to bf16 / fp16; fp32 stays;
  * the fp64 view of an input is the exact upcast of the stored value, so
    the oracle sees the numbers the GPU sees, not the pre-rounding samples.

Layouts are row-major contiguous: Q/out ``[B,Hq,Lq,d]``, K/V ``[B,Hkv,Lk,d]``,
dense mask ``[Lq,Lk]`` fp32, zero_hold ``[B,Hkv,Lk]`` fp32.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import numpy as np

DTYPE_CODES = {"fp32": 0, "fp16": 1, "bf16": 2}
MASK_CODES = {"none": 0, "causal": 1, "window": 2, "dense": 3, "topk": 4}


# ---------------------------------------------------------------- rounding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """The array whose bytes the GPU receives (uint16 bits for bf16)."""
    if dtype == "fp32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def storage_to_f64(s: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(s)
    return s.astype(np.float64)


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# ------------------------------------------------------------------ problem
@dataclass
class Problem:
    """One attention-forward call: sizes, flags and stored inputs."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    d: int
    dtype: str
    mask_kind: str
    scale: float                      # the fp32 value passed across the ABI
    window_left: int = 0
    keep_k: int = 0
    q: np.ndarray = None              # storage arrays
    k: np.ndarray = None
    v: np.ndarray = None
    mask: np.ndarray | None = None    # fp32 [Lq, Lk]
    zero_hold: np.ndarray | None = None   # fp32 [B, Hkv, Lk]
    meta: dict = field(default_factory=dict)

    def f64(self, name: str) -> np.ndarray:
        return storage_to_f64(getattr(self, name), self.dtype)

    @property
    def scale64(self) -> float:
        return float(np.float32(self.scale))


def default_scale(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


def draw(seed: int, shapes, mult: float = 1.0):
    rng = np.random.default_rng(seed)
    out = []
    for s in shapes:
        x = rng.standard_normal(s, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)   # exact for powers of two
        out.append(x)
    return out


def make_problem(name, B, Hq, Hkv, Lq, Lk, d, dtype, mask_kind, seed, *, scale=None,
                 window_left=0, keep_k=0, mask=None, with_zero_hold=False, mult=1.0,
                 kv_keys=None) -> Problem:
    """Draw q, k, v (and zero_hold) in that order from ``seed``.

    ``kv_keys`` draws K/V (and zero_hold) with ``kv_keys`` keys and keeps the first ``Lk``;
    it lets a shorter-cache variant reuse a longer cache's data.
    """
    Lk_draw = Lk if kv_keys is None else kv_keys
    shapes = [(B, Hq, Lq, d), (B, Hkv, Lk_draw, d), (B, Hkv, Lk_draw, d)]
    if with_zero_hold:
        shapes.append((B, Hkv, Lk_draw))
    arrs = draw(seed, shapes, mult)
    q32, k32, v32 = arrs[:3]
    k32 = np.ascontiguousarray(k32[:, :, :Lk])
    v32 = np.ascontiguousarray(v32[:, :, :Lk])
    zh = np.ascontiguousarray(arrs[3][:, :, :Lk]) if with_zero_hold else None
    p = Problem(name=name, B=B, Hq=Hq, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d, dtype=dtype,
                mask_kind=mask_kind, scale=default_scale(d) if scale is None else float(np.float32(scale)),
                window_left=window_left, keep_k=keep_k,
                q=to_storage(q32, dtype), k=to_storage(k32, dtype), v=to_storage(v32, dtype),
                mask=mask, zero_hold=zh)
    p.meta["seed"] = seed
    return p


def window_dense_mask(Lq: int, Lk: int, first_pos: int, window: int) -> np.ndarray:
    """fp32 [Lq, Lk] additive mask: 0 on keys pos-window..pos (inclusive), -inf elsewhere,
    for query rows at absolute positions first_pos .. first_pos+Lq-1 (an input, built
    by the caller of the attention call the way the ExecuTorch page describes)."""
    m = np.full((Lq, Lk), -np.inf, dtype=np.float32)
    for i in range(Lq):
        pos = first_pos + i
        lo, hi = max(0, pos - window), min(Lk - 1, pos)
        if hi >= lo:
            m[i, lo:hi + 1] = 0.0
    return m


# ------------------------------------------------------------ varlen / paged problems
@dataclass
class PagedProblem:
    """One attention call over a batch of sequences of different lengths.

    Queries are packed token-major ``[total_q, Hq, d]`` with ``cu_seqlens_q``; sequence
    ``s`` has ``cu_seqlens_k[s+1] - cu_seqlens_k[s]`` keys. With ``page_size > 0`` K/V are
    a paged cache ``[num_pages, page_size, Hkv, d]`` addressed through ``block_table``
    ``[S, max_pages]`` (int32, unused entries 0); with ``page_size == 0`` they are packed
    ``[total_k, Hkv, d]`` at the ``cu_seqlens_k`` offsets. ``k_new``/``v_new``
    ``[total_q, Hkv, d]`` (two-source form) hold each sequence's last ``Lq`` keys, and the
    cache then holds only the first ``Lk - Lq``.
    """
    name: str
    Hq: int
    Hkv: int
    d: int
    dtype: str
    mask_kind: str
    scale: float
    page_size: int
    window_left: int = 0
    cu_seqlens_q: np.ndarray = None
    cu_seqlens_k: np.ndarray = None
    block_table: np.ndarray | None = None
    q: np.ndarray = None
    k: np.ndarray = None
    v: np.ndarray = None
    k_new: np.ndarray | None = None
    v_new: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    def f64(self, name: str):
        a = getattr(self, name)
        return None if a is None else storage_to_f64(a, self.dtype)

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens_q.size - 1)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q)

    @property
    def k_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_k)

    @property
    def max_seqlen_q(self) -> int:
        return int(self.q_lens.max(initial=0))

    @property
    def max_seqlen_k(self) -> int:
        return int(self.k_lens.max(initial=0))

    @property
    def kv_rows(self) -> int:
        """Leading extent of K/V: pages when paged, rows when packed."""
        return int(self.k.shape[0])

    @property
    def two_source(self) -> bool:
        return self.k_new is not None


def make_paged_problem(name, q_lens, k_lens, Hq, Hkv, d, dtype, mask_kind, seed, *, page_size=16,
                       two_source=False, window_left=0, spare_pages=2, mult=1.0, scale=None) -> PagedProblem:
    """Draw q, K/V storage, (k_new, v_new), then the page permutation, from ``seed``.

    Physical pages are a random permutation of the pool (plus ``spare_pages`` pages no
    sequence uses), so logically consecutive pages are scattered as in a serving cache.
    """
    q_lens = np.asarray(q_lens, dtype=np.int64)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    S = q_lens.size
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    cached = np.maximum(k_lens - q_lens, 0) if two_source else k_lens
    rng = np.random.default_rng(seed)

    def normal(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        return x

    q32 = normal((total_q, Hq, d))
    if page_size > 0:
        pages = (cached + page_size - 1) // page_size
        num_pages = int(pages.sum()) + spare_pages
        kv_shape = (num_pages, page_size, Hkv, d)
    else:
        kv_shape = (total_k, Hkv, d)
    k32, v32 = normal(kv_shape), normal(kv_shape)
    kn32 = vn32 = None
    if two_source:
        kn32, vn32 = normal((total_q, Hkv, d)), normal((total_q, Hkv, d))
    table = None
    if page_size > 0:
        perm = rng.permutation(num_pages).astype(np.int32)
        table = np.zeros((S, max(1, int(pages.max(initial=0)))), dtype=np.int32)
        nxt = 0
        for s in range(S):
            table[s, :pages[s]] = perm[nxt:nxt + pages[s]]
            nxt += int(pages[s])
    p = PagedProblem(name=name, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, mask_kind=mask_kind,
                     scale=default_scale(d) if scale is None else float(np.float32(scale)),
                     page_size=page_size, window_left=window_left, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                     block_table=table, q=to_storage(q32, dtype), k=to_storage(k32, dtype),
                     v=to_storage(v32, dtype),
                     k_new=None if kn32 is None else to_storage(kn32, dtype),
                     v_new=None if vn32 is None else to_storage(vn32, dtype))
    p.meta["seed"] = seed
    return p


def serving_lengths(seed, n_prefill, prefill_q, prefill_ctx, n_decode, decode_ctx):
    """A mixed serving batch: ``n_prefill`` chunks of ``prefill_q`` new tokens on top of
    contexts drawn uniformly from ``prefill_ctx = (lo, hi)``, then ``n_decode`` single-token
    steps with contexts drawn log-uniformly from ``decode_ctx = (lo, hi)``. Returns
    (q_lens, k_lens); key counts include the new tokens."""
    rng = np.random.default_rng(seed)
    pc = rng.integers(prefill_ctx[0], prefill_ctx[1] + 1, size=n_prefill)
    lo, hi = np.log(decode_ctx[0]), np.log(decode_ctx[1])
    dc = np.exp(rng.uniform(lo, hi, size=n_decode)).astype(np.int64)
    q_lens = np.concatenate([np.full(n_prefill, prefill_q), np.ones(n_decode, dtype=np.int64)])
    k_lens = np.concatenate([pc + prefill_q, dc + 1])
    return q_lens.astype(np.int64), k_lens.astype(np.int64)


def paged_config(name: str) -> PagedProblem:
    """Varlen / paged workloads: a small mixed batch with the edge cases, and a serving batch."""
    if name == "v1":
        # decode step, prefill chunk over a context, a one-key sequence, a plain prefill,
        # a sequence with no queries, more queries than keys, and one with no keys at all
        q_lens = [1, 37, 1, 130, 0, 5, 3]
        k_lens = [300, 200, 1, 130, 50, 3, 0]
        return make_paged_problem("v1 small mixed varlen, paged 16", q_lens, k_lens, 8, 2, 128, "bf16",
                                  "causal", 61, page_size=16)
    if name == "serve":
        q_lens, k_lens = serving_lengths(62, 4, 512, (1024, 4096), 60, (1024, 16384))
        return make_paged_problem("serving batch: 4 prefill chunks of 512 + 60 decode steps, paged 16",
                                  q_lens, k_lens, 32, 8, 128, "bf16", "causal", 63, page_size=16)
    raise KeyError(name)


# ------------------------------------------------------------ named configs
def config(name: str) -> Problem:
    """The five workloads (and their variants) at full size."""
    if name == "c1":
        return make_problem("c1 tiny causal fp32", 1, 2, 2, 128, 128, 64, "fp32", "causal", 1, scale=0.125)
    if name == "c2":
        return make_problem("c2 dense window-60 GQA", 4, 32, 8, 16, 700, 128, "bf16", "dense", 2,
                            mask=window_dense_mask(16, 700, 560, 60))
    if name == "c2b":
        return make_problem("c2b fully masked rows", 4, 32, 8, 4, 700, 128, "bf16", "dense", 21,
                            mask=np.full((4, 700), -np.inf, dtype=np.float32))
    if name == "c2c":
        return make_problem("c2c inclusive window 0", 4, 32, 8, 4, 700, 128, "bf16", "dense", 22,
                            mask=window_dense_mask(4, 700, 572, 0))
    if name == "c2w":
        return make_problem("c2w window kind, W=60, Lk=576", 4, 32, 8, 16, 576, 128, "bf16", "window", 2,
                            window_left=60, kv_keys=700)
    if name == "c3p":
        return make_problem("c3 prefill bottom-right causal", 8, 32, 8, 512, 4096, 128, "bf16", "causal", 3)
    if name == "c3d":
        return make_problem("c3 decode split-KV", 16, 32, 8, 1, 32768, 128, "bf16", "causal", 33)
    c4 = {"c4_d64_bf16": (64, "bf16", 41), "c4_d64_fp16": (64, "fp16", 42),
          "c4_d128_bf16": (128, "bf16", 43), "c4_d128_fp16": (128, "fp16", 44)}
    if name in c4:
        d, dt, seed = c4[name]
        return make_problem(f"c4 long causal d{d} {dt}", 4, 16, 16, 8192, 8192, d, dt, "causal", seed, mult=0.5)
    if name == "c5":
        return make_problem("c5 dynamic top-k", 2, 16, 16, 4096, 4096, 128, "bf16", "topk", 5,
                            keep_k=1024, with_zero_hold=True)
    raise KeyError(name)


CONFIG_NAMES = ["c1", "c2", "c2b", "c2c", "c2w", "c3p", "c3d",
                "c4_d64_bf16", "c4_d64_fp16", "c4_d128_bf16", "c4_d128_fp16", "c5"]


# ------------------------------------------------------------ attn_fwd_ex workloads
def alibi_slopes(H: int) -> np.ndarray:
    """fp32 [H]: the geometric slopes 2^(-8 (h+1) / H), the usual ALiBi choice (an input
    here: the pages name the slopes argument without giving values)."""
    return (2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32)


def per_head_window_mask(B: int, H: int, Lq: int, Lk: int, first_pos: int, base_window: int) -> np.ndarray:
    """fp32 [1, H, Lq, Lk]: head h sees keys pos-(base_window - h)..pos (a window that
    narrows with the head), the same for every batch."""
    m = np.stack([window_dense_mask(Lq, Lk, first_pos, max(base_window - h, 0)) for h in range(H)])
    return m[None]


EX_NAMES = ["c3p_alibi_softcap", "c3p_kv_blhd", "c3d_kv_blhd", "c5_noncausal", "c2_per_head_mask"]


def ex_config(name: str):
    """Workloads of attn_fwd_ex: one of the five configurations with a general layout, a
    score modifier, a top-k variant or a per-head mask. Returns (problem, options) with
    options: layout ("bhld" or "blhd" for q, k, v and out), alibi (fp32 [Hq] or None),
    softcap (float), topk_causal (bool), mask (fp32 array broadcasting to [B,Hq,Lq,Lk]
    or None)."""
    opts = {"layout": "bhld", "alibi": None, "softcap": 0.0, "topk_causal": True, "mask": None}
    if name == "c3p_alibi_softcap":
        p = config("c3p")
        opts.update(alibi=alibi_slopes(p.Hq), softcap=30.0)
    elif name == "c3p_kv_blhd":
        p = config("c3p")
        opts.update(layout="blhd")
    elif name == "c3d_kv_blhd":
        p = config("c3d")
        opts.update(layout="blhd")
    elif name == "c5_noncausal":
        p = config("c5")
        opts.update(topk_causal=False)
    elif name == "c2_per_head_mask":
        p = config("c2")
        # the rows sit at positions 560..575 of the 700-key cache, as in c2
        opts.update(mask=per_head_window_mask(p.B, p.Hq, p.Lq, p.Lk, 560, 60))
    else:
        raise KeyError(name)
    p.name = f"{p.name} + {name.split('_', 1)[1].replace('_', ' ')}"
    return p, opts
