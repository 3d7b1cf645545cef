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
