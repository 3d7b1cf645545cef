"""Benchmark of the masked attention forward on one MI355X.

Headline (the JSON line's ``value``): causal prefill with past keys, bottom-right
aligned -- B=8, Hq=32, Hkv=8, Lq=512, Lk=4096, d=128, bf16 -- in TFLOP/s of
algorithmic work (4*d flops per visible (row, key) pair). One step is one
``attn_fwd`` call on that batch, inputs resident in HBM before timing starts.

The same line carries:
  roofline      the prefill kernel's achieved TFLOP/s against the bf16 dense MFMA peak,
                timed with events on the stream the library launches on;
  cpu_baseline  the fp64 oracle on every head of the same workload, timed on this host;
  configs       every other workload (decode GB/s, long causal, top-k, dense window,
                tiny fp32), the paged serving batch of attn_fwd_varlen (plain, and with ALiBi +
                softcap) and the attn_fwd_ex
                workloads (transposed KV cache, ALiBi + softcap, non-causal top-k, per-head
                mask; each with the plain call's time on the same data) and the backward
                (attn_bwd) on the long causal and prefill workloads; the five
                configurations also carry the oracle timed on this host (c4: 4 of its 64
                heads, scaled up and labelled extrapolated);
  decode        the decode workload's GB/s, also as a fraction of a plain read stream
                (attn_read_stream) measured in the same run. Parity at these
                sizes is the GPU tests' job (tests/test_gpu_parity.py, test_gpu_varlen.py,
                test_gpu_ex.py, test_gpu_bwd.py);
                the benchmark only times.

Usage: python bench.py [--steps K] [--warmup W] [--only NAME] [--no-cpu-baseline]
                       [--no-configs] [--copy-calibration BYTES]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (prefill, % MFMA peak); decode KV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk/CU (published 2.5 PFLOP/s dense)
PEAK_HBM_GBS = 8000.0       # 8 TB/s HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs(p) -> int:
    """(row, key) pairs the mask leaves visible, summed over batch and heads."""
    Lq, Lk = p.Lq, p.Lk
    pos = np.arange(Lq) + (Lk - Lq)
    if p.mask_kind == "none":
        per = Lq * Lk
    elif p.mask_kind == "causal":
        per = int(np.clip(pos + 1, 0, Lk).sum())
    elif p.mask_kind == "window":
        hi = np.clip(pos + 1, 0, Lk)
        lo = np.clip(pos - p.window_left, 0, Lk)
        per = int(np.maximum(hi - lo, 0).sum())
    elif p.mask_kind == "dense":
        per = int(np.isfinite(p.mask).sum())
    elif p.mask_kind == "topk":
        per = int(np.minimum(np.clip(pos + 1, 0, Lk), p.keep_k).sum())
    else:
        raise ValueError(p.mask_kind)
    return per * p.B * p.Hq


def causal_pairs(p) -> int:
    pos = np.arange(p.Lq) + (p.Lk - p.Lq)
    return int(np.clip(pos + 1, 0, p.Lk).sum()) * p.B * p.Hq


def algorithmic_bytes(p) -> int:
    """Q + out + LSE + the distinct K/V rows some row can see (+ mask / zero_hold)."""
    es = 4 if p.dtype == "fp32" else 2
    q = p.B * p.Hq * p.Lq * p.d * es
    lse = p.B * p.Hq * p.Lq * 4
    pos = np.arange(p.Lq) + (p.Lk - p.Lq)
    if p.mask_kind in ("causal", "topk"):
        keys = min(p.Lk, int(pos.max()) + 1) if pos.max() >= 0 else 0
    elif p.mask_kind == "window":
        keys = min(p.Lk, int(pos.max()) + 1) - max(0, int(pos.min()) - p.window_left)
    elif p.mask_kind == "dense":
        keys = int(np.isfinite(p.mask).any(axis=0).sum())
    else:
        keys = p.Lk
    kv = 2 * p.B * p.Hkv * keys * p.d * es
    extra = 0
    if p.mask_kind == "dense":
        extra = p.mask.nbytes
    if p.mask_kind == "topk":
        extra = p.zero_hold.nbytes
    return int(2 * q + lse + kv + extra)


class Runner:
    """Device copies of one problem and a bound attn_fwd call."""

    def __init__(self, p):
        import torch
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        self.p = p
        dev = "cuda"

        def t(a):
            if p.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self.q, self.k, self.v = t(p.q), t(p.k), t(p.v)
        self.mask = torch.from_numpy(p.mask).to(dev) if p.mask is not None else None
        self.zh = torch.from_numpy(p.zero_hold).to(dev) if p.zero_hold is not None else None
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((p.B, p.Hq, p.Lq), dtype=torch.float32, device=dev)

    def __call__(self):
        import masked_flashattention_forward_amd as mfa
        p = self.p
        mfa.attn_fwd(self.q, self.k, self.v, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left,
                     mask=self.mask if p.mask_kind == "dense" else None,
                     zero_hold=self.zh if p.mask_kind == "topk" else None, keep_k=p.keep_k,
                     out=self.out, lse=self.lse)


WARM_MS = 200.0  # time-based warm-up before any timed call: clocks ramp before timing


def warm(fn, min_calls: int = 3, min_ms: float = WARM_MS) -> float:
    """Call fn until at least ``min_calls`` calls and ``min_ms`` of wall time have passed
    (synchronised); returns the warm-up time in ms."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def event_times_ms(fn, iters: int) -> np.ndarray:
    """Per-call durations from a HIP event pair around each call, recorded on torch's
    current stream, which is the stream the library launches on."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def time_calls(fn, iters: int = 20) -> dict:
    """Time-based warm-up, then per-call event durations: mean, median and min in us."""
    w = warm(fn)
    t = event_times_ms(fn, iters)
    return {"us": round(float(t.mean()) * 1e3, 2), "us_median": round(float(np.median(t)) * 1e3, 2),
            "us_min": round(float(t.min()) * 1e3, 2), "iters": iters, "warmup_ms": round(w, 1)}


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the oracle baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_oracle(p, heads=None, label="") -> dict:
    """The fp64 oracle, as it stands, timed on this host's cores: every (batch, head) of the
    workload, or only ``heads`` (then scaled up to the whole workload and labelled
    extrapolated). Input conversion to fp64 is outside the timed region; the result is in
    TFLOP/s of algorithmic work (4*d flops per visible (row, key) pair)."""
    import oracle
    import synth
    pairs = [(b, h) for b in range(p.B) for h in range(p.Hq)]
    sample = pairs if heads is None else heads
    G = p.Hq // p.Hkv
    elapsed = 0.0
    mask = None if p.mask is None else p.mask.astype(np.float64)
    for b in sorted({b for b, _ in sample}):
        hs = [h for bb, h in sample if bb == b]
        gs = sorted({h // G for h in hs})
        # one batch element at a time; only the KV heads the sampled query heads read
        q = synth.storage_to_f64(p.q[b:b + 1], p.dtype)
        k = np.zeros((1, p.Hkv, p.Lk, p.d))
        v = np.zeros((1, p.Hkv, p.Lk, p.d))
        k[:, gs] = synth.storage_to_f64(p.k[b:b + 1, gs], p.dtype)
        v[:, gs] = synth.storage_to_f64(p.v[b:b + 1, gs], p.dtype)
        zh = None if p.zero_hold is None else p.zero_hold[b:b + 1].astype(np.float64)
        t0 = time.perf_counter()
        oracle.attention_ref(q, k, v, p.scale64, p.mask_kind, window_left=p.window_left, mask=mask,
                             zero_hold=zh, keep_k=p.keep_k, heads=[(0, h) for h in hs])
        elapsed += time.perf_counter() - t0
    frac = len(sample) / len(pairs)
    flops = 4.0 * p.d * visible_pairs(p)
    dt = elapsed / frac
    res = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
           "cpu": cpu_model(), "seconds": round(dt, 3)}
    if heads is None:
        res["sample"] = f"fp64 oracle on all {len(pairs)} (b,h) heads of {label or p.name}, {elapsed:.1f} s"
    else:
        res["sample"] = (f"fp64 oracle on {len(sample)} of {len(pairs)} (b,h) heads of {label or p.name} "
                         f"(all {p.Lq} rows each), {elapsed:.1f} s, scaled x{len(pairs) / len(sample):g}: "
                         f"extrapolated")
        res["extrapolated"] = True
    log(f"cpu oracle {label or p.name}: {json.dumps(res)}")
    return res


def c4_oracle_heads(p, n=4, seed=4):
    rng = np.random.default_rng(seed)
    pairs = [(b, h) for b in range(p.B) for h in range(p.Hq)]
    return sorted(pairs[int(i)] for i in rng.choice(len(pairs), size=n, replace=False))


def bench_config(name, iters=20, with_oracle=False):
    import synth
    p = synth.config(name)
    r = Runner(p)
    import torch
    tm = time_calls(r, iters)
    ms = tm["us"] / 1e3
    res = {"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Lq": p.Lq, "Lk": p.Lk, "d": p.d,
           "dtype": p.dtype, "mask": p.mask_kind, **tm}
    flops = 4.0 * p.d * visible_pairs(p)
    byts = algorithmic_bytes(p)
    res["tflops"] = round(flops / ms / 1e9, 2)
    res["pct_mfma_peak"] = round(100 * flops / ms / 1e9 / PEAK_BF16_TFLOPS, 2)
    res["tflops_median"] = round(flops / tm["us_median"] / 1e6, 2)
    res["gbs"] = round(byts / ms / 1e6, 1)
    res["pct_hbm_peak"] = round(100 * byts / ms / 1e6 / PEAK_HBM_GBS, 2)
    if p.mask_kind == "topk":
        cf = 4.0 * p.d * causal_pairs(p)
        res["tflops_causal_tiles"] = round(cf / ms / 1e9, 2)
        import masked_flashattention_forward_amd as mfa
        zt = r.zh
        res["dynamic_mask_topk_us"] = time_calls(lambda: mfa.dynamic_mask_topk(zt, p.Lq, p.keep_k), iters)["us"]
    import masked_flashattention_forward_amd as mfa
    res["plan"] = mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, p.mask_kind, p.window_left, p.keep_k,
                           synth.DTYPE_CODES[p.dtype])
    del r
    torch.cuda.empty_cache()
    log(f"{name}: {json.dumps(res)}")
    if with_oracle:
        heads = c4_oracle_heads(p) if name.startswith("c4") else None
        res["cpu_baseline"] = cpu_oracle(p, heads=heads, label=name)
    return res


def bench_topk_select(B=2, H=16, L=32768, keep_k=1024, iters=10) -> dict:
    """dynamic_mask_topk alone over a long cache (c5's selection at L keys and L query
    rows, zero_hold N(0,1) from seed 5): ranks by chunk sort and run merge, then the
    per-row thresholds."""
    import torch
    import masked_flashattention_forward_amd as mfa
    zh = torch.from_numpy(np.random.default_rng(5).standard_normal((B, H, L), dtype=np.float32)).cuda()
    tm = time_calls(lambda: mfa.dynamic_mask_topk(zh, L, keep_k), iters)
    res = {"workload": f"dynamic_mask_topk zero_hold [{B},{H},{L}], {L} query rows, keep {keep_k}", **tm}
    del zh
    torch.cuda.empty_cache()
    log(f"topk select {L}: {json.dumps(res)}")
    return res


def bench_read_stream(nbytes: int, iters=20) -> dict:
    """The plain HBM read stream (attn_read_stream) over a buffer the size of the decode
    workload's K and V, with and without the non-temporal hint: the practical ceiling the
    decode kernel's bandwidth is reported against."""
    import torch
    import masked_flashattention_forward_amd as mfa
    buf = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    out = {"bytes": nbytes}
    for nt in (False, True):
        sink = torch.empty((nbytes + mfa.READ_STREAM_CHUNK - 1) // mfa.READ_STREAM_CHUNK, dtype=torch.int32,
                           device="cuda")
        tm = time_calls(lambda: mfa.read_stream(buf, nontemporal=nt, sink=sink), iters)
        key = "nontemporal" if nt else "plain"
        out[key] = {"us": tm["us"], "us_median": tm["us_median"], "gbs": round(nbytes / tm["us"] / 1e3, 1)}
    out["best_gbs"] = max(out["plain"]["gbs"], out["nontemporal"]["gbs"])
    del buf
    torch.cuda.empty_cache()
    log(f"read stream: {json.dumps(out)}")
    return out


def bench_ex_config(name, iters=20):
    """One attn_fwd_ex workload (synth.ex_config): a general layout, score modifiers, a
    top-k variant or a per-head mask on one of the five configurations. Reports the time
    next to that of the plain call on the same data, so the line shows what the option
    costs."""
    import torch
    import masked_flashattention_forward_amd as mfa
    import synth
    p, o = synth.ex_config(name)
    r = Runner(p)

    def lay(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2) if o["layout"] == "blhd" else t

    q, k, v = lay(r.q), lay(r.k), lay(r.v)
    out = lay(torch.empty_like(r.q))
    mask = None
    if o["mask"] is not None:
        mask = torch.from_numpy(o["mask"]).cuda()
    elif p.mask_kind == "dense":
        mask = r.mask
    sl = None if o["alibi"] is None else torch.from_numpy(o["alibi"]).cuda()

    def call():
        mfa.attn_fwd_ex(q, k, v, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left, mask=mask,
                        zero_hold=r.zh, keep_k=p.keep_k, topk_causal=o["topk_causal"], alibi_slopes=sl,
                        softcap=o["softcap"], out=out, lse=r.lse)

    tm = time_calls(call, iters)
    tm_plain = time_calls(r, iters)
    ms, ms_plain = tm["us"] / 1e3, tm_plain["us"] / 1e3
    if o["mask"] is not None:
        pairs = int(np.isfinite(np.broadcast_to(o["mask"], (p.B, p.Hq, p.Lq, p.Lk))).sum())
    elif p.mask_kind == "topk" and not o["topk_causal"]:
        pairs = p.B * p.Hq * p.Lq * min(p.keep_k, p.Lk)
    else:
        pairs = visible_pairs(p)
    flops = 4.0 * p.d * pairs
    byts = algorithmic_bytes(p) + (0 if o["mask"] is None else o["mask"].nbytes)
    res = {"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Lq": p.Lq, "Lk": p.Lk, "d": p.d,
           "dtype": p.dtype, "mask": p.mask_kind, "layout": o["layout"], "alibi": o["alibi"] is not None,
           "softcap": o["softcap"], "topk_causal": o["topk_causal"], "per_head_mask": o["mask"] is not None,
           "us": round(ms * 1e3, 2), "us_median": tm["us_median"], "us_min": tm["us_min"],
           "us_plain_call": round(ms_plain * 1e3, 2),
           "tflops": round(flops / ms / 1e9, 2), "pct_mfma_peak": round(100 * flops / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
           "gbs": round(byts / ms / 1e6, 1), "pct_hbm_peak": round(100 * byts / ms / 1e6 / PEAK_HBM_GBS, 2)}
    del r, q, k, v, out, mask
    torch.cuda.empty_cache()
    log(f"{name}: {json.dumps(res)}")
    return res


def bench_bwd_config(name, iters=10):
    """attn_bwd on one of the configurations: the forward runs once for out and lse, then
    the backward call (rowsum, dK/dV and dQ kernels) is timed. Algorithmic work: the five
    products of the backward, 10*d flops per visible (row, key) pair (the kernels execute
    14*d: S and dP are computed in both the dK/dV and the dQ kernel)."""
    import torch
    import masked_flashattention_forward_amd as mfa
    import synth
    p = synth.config(name)
    r = Runner(p)
    r()
    dout = torch.randn(r.q.shape, generator=torch.Generator(device="cuda").manual_seed(7), device="cuda",
                       dtype=torch.float32).to(r.q.dtype)
    dq, dk, dv = torch.empty_like(r.q), torch.empty_like(r.k), torch.empty_like(r.v)
    kw = dict(scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left,
              mask=r.mask if p.mask_kind == "dense" else None, zero_hold=r.zh if p.mask_kind == "topk" else None,
              keep_k=p.keep_k, dq=dq, dk=dk, dv=dv)

    def call():
        mfa.attn_bwd(r.q, r.k, r.v, r.out, r.lse, dout, **kw)

    tm = time_calls(call, iters)
    tm_fwd = time_calls(r, iters)
    ms, ms_fwd = tm["us"] / 1e3, tm_fwd["us"] / 1e3
    pairs = visible_pairs(p)
    flops = 10.0 * p.d * pairs
    res = {"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Lq": p.Lq, "Lk": p.Lk, "d": p.d,
           "dtype": p.dtype, "mask": p.mask_kind, "us": round(ms * 1e3, 2), "us_median": tm["us_median"],
           "us_min": tm["us_min"], "us_forward": round(ms_fwd * 1e3, 2),
           "tflops": round(flops / ms / 1e9, 2), "pct_mfma_peak": round(100 * flops / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
           "tflops_executed": round(1.4 * flops / ms / 1e9, 2)}
    del r, dout, dq, dk, dv
    torch.cuda.empty_cache()
    log(f"{name} backward: {json.dumps(res)}")
    return res


def paged_pairs_and_keys(p):
    """Visible (row, key) pairs over all query heads, and distinct visible keys per KV
    head, of a varlen problem (each sequence bottom-right aligned)."""
    pairs = keys = 0
    for Lq, Lk in zip(p.q_lens.tolist(), p.k_lens.tolist()):
        if Lq == 0 or (p.two_source and Lk < Lq):
            continue
        pos = np.arange(Lq) + (Lk - Lq)
        hi = np.clip(pos + 1, 0, Lk) if p.mask_kind != "none" else np.full(Lq, Lk)
        lo = np.clip(pos - p.window_left, 0, Lk) if p.mask_kind == "window" else np.zeros(Lq, dtype=np.int64)
        pairs += int(np.maximum(hi - lo, 0).sum())
        keys += int(max(0, hi.max() - lo.min()))
    return pairs * p.Hq, keys


def bench_paged_config(name, iters=20, modifiers=False):
    """attn_fwd_varlen on a paged serving batch: time, algorithmic TFLOP/s and GB/s, and
    the fraction of the roofline time max(flops / MFMA peak, bytes / HBM peak). With
    ``modifiers`` the call also applies ALiBi (the geometric slopes) and softcap 30."""
    import torch
    import masked_flashattention_forward_amd as mfa
    import synth
    p = synth.paged_config(name)

    def t(a):
        if a is None:
            return None
        if p.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    q, k, v, kn, vn = (t(getattr(p, n)) for n in ("q", "k", "v", "k_new", "v_new"))
    cu_q = torch.from_numpy(p.cu_seqlens_q).cuda()
    cu_k = torch.from_numpy(p.cu_seqlens_k).cuda()
    bt = None if p.block_table is None else torch.from_numpy(p.block_table).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((p.total_q, p.Hq), dtype=torch.float32, device="cuda")
    sl = torch.from_numpy(synth.alibi_slopes(p.Hq)).cuda() if modifiers else None
    cap = 30.0 if modifiers else 0.0

    def call():
        mfa.attn_fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q=p.max_seqlen_q, max_seqlen_k=p.max_seqlen_k,
                            block_table=bt, k_new=kn, v_new=vn, scale=p.scale, mask_kind=p.mask_kind,
                            window_left=p.window_left, alibi_slopes=sl, softcap=cap, out=out, lse=lse)

    tm = time_calls(call, iters)
    ms = tm["us"] / 1e3
    pairs, keys = paged_pairs_and_keys(p)
    flops = 4.0 * p.d * pairs
    es = 2
    byts = 2 * p.total_q * p.Hq * p.d * es + p.total_q * p.Hq * 4 + 2 * p.Hkv * keys * p.d * es
    t_roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9)) * 1e3
    res = {"workload": p.name, "num_seqs": p.num_seqs, "total_q": p.total_q, "total_k": int(p.k_lens.sum()),
           "Hq": p.Hq, "Hkv": p.Hkv, "d": p.d, "page_size": p.page_size, "dtype": p.dtype, "mask": p.mask_kind,
           "alibi": modifiers, "softcap": cap,
           "us": round(ms * 1e3, 2), "us_median": tm["us_median"], "us_min": tm["us_min"],
           "tflops": round(flops / ms / 1e9, 2),
           "pct_mfma_peak": round(100 * flops / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
           "gbs": round(byts / ms / 1e6, 1), "pct_hbm_peak": round(100 * byts / ms / 1e6 / PEAK_HBM_GBS, 2),
           "roofline_time_frac": round(t_roof / ms, 4)}
    del q, k, v, kn, vn, out, lse
    torch.cuda.empty_cache()
    log(f"{name}: {json.dumps(res)}")
    return res


def measured_traffic(kernel_key: str):
    """HBM bytes per dispatch from the committed counter runs (profiles/traffic.json), or
    None when the kernel sources changed since those counters were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["kernels"][kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    m = hashlib.sha256()
    for f in rec["sources"]:
        m.update(open(os.path.join(ROOT, "masked_flashattention_forward_amd", "csrc", f), "rb").read())
    return rec["traffic_bytes"] if m.hexdigest() == rec["source_sha256"] else None


def copy_calibration(nbytes: int, iters: int):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(iters):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copied {nbytes} bytes x {iters}")


def headline_roofline(name, p, plan, flops, kern, warm_ms):
    """The roofline object of the timed workload: MFMA-bound (TFLOP/s of the visible pairs)
    on the prefill path, HBM-bound (algorithmic bytes) on the split-KV decode path, with
    the calibrated HBM traffic when the committed counters belong to this workload and the
    current kernel sources."""
    kern_ms = float(kern.mean())
    med_ms = float(np.median(kern))
    nbytes = algorithmic_bytes(p)
    common = {"algorithmic_bytes": nbytes, "avg_kernel_us": round(kern_ms * 1e3, 2),
              "median_kernel_us": round(med_ms * 1e3, 2), "min_kernel_us": round(float(kern.min()) * 1e3, 2),
              "warmup_ms": round(warm_ms, 1)}
    if plan["path"] == "splitkv_decode":
        achieved = nbytes / kern_ms / 1e6
        return {"bound": "hbm", "kernel": f"decode_kernel<{p.dtype},{p.d},{p.mask_kind}> + lse_merge_kernel",
                "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic("decode_kernel<bf16,128,causal> c3 decode") if name == "c3d" else None,
                **common, "frac_at_median": round(nbytes / med_ms / 1e6 / PEAK_HBM_GBS, 4)}
    achieved = flops / kern_ms / 1e9
    return {"bound": "mfma", "kernel": f"prefill_kernel<{p.dtype},{p.d},{plan['block_n']},{p.mask_kind}>",
            "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("prefill_kernel<bf16,128,64,causal> c3 prefill") if name == "c3p" else None,
            **common, "frac_at_median": round(flops / med_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}


FWD_CONFIGS = ("c3d", "c4_d128_bf16", "c4_d64_bf16", "c4_d128_fp16", "c4_d64_fp16", "c5", "c2", "c2w", "c1")
BWD_CONFIGS = ("c4_d128_bf16", "c4_d64_bf16", "c4_d128_fp16", "c4_d64_fp16", "c3p")


def config_entries(oracle_on):
    """The per-configuration entries of the JSON line in their order: (key, progress label,
    function that measures it)."""
    import synth
    out = [(n, f"config {n}", lambda n=n: bench_config(n, with_oracle=oracle_on and n != "c2w"))
           for n in FWD_CONFIGS]
    out.append(("c5_topk_select_32k", "config c5 selection at 32768 keys", bench_topk_select))
    out.append(("serve", "config serve (paged varlen)", lambda: bench_paged_config("serve")))
    out.append(("serve_alibi_softcap", "config serve with ALiBi + softcap (paged varlen)",
                lambda: bench_paged_config("serve", modifiers=True)))
    out += [(n, f"config {n} (attn_fwd_ex)", lambda n=n: bench_ex_config(n)) for n in synth.EX_NAMES]
    out += [(f"{n}_bwd", f"config {n} (attn_bwd)", lambda n=n: bench_bwd_config(n)) for n in BWD_CONFIGS]
    return out


def config_entry_names():
    return [key for key, _, _ in config_entries(False)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--only", default="c3p", help="headline workload name (see synth.CONFIG_NAMES)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--configs", default="",
                    help="comma-separated subset of the per-configuration entries to run (default: all of them)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (--gpus {args.gpus} requested)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return
    wanted = [n for n in args.configs.split(",") if n]
    unknown = sorted(set(wanted) - set(config_entry_names()))
    if unknown:
        print(f"unknown --configs entries: {', '.join(unknown)} (known: {', '.join(config_entry_names())})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import masked_flashattention_forward_amd as mfa
    import synth
    mfa.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    log(f"generating {args.only}")
    p = synth.config(args.only)
    r = Runner(p)
    # warm-up: the W untimed steps, continued until at least 200 ms of wall time have
    # passed so that the clocks have ramped before the timed steps
    warm_ms = warm(r, min_calls=max(args.warmup, 1))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        r()
        b.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kern = np.array([a.elapsed_time(b) for a, b in ev])
    kern_ms = float(kern.mean())
    flops = 4.0 * p.d * visible_pairs(p)
    value = flops / wall_ms / 1e9
    achieved = flops / kern_ms / 1e9
    plan = mfa.plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.d, p.mask_kind, p.window_left, p.keep_k,
                    synth.DTYPE_CODES[p.dtype])
    log(f"headline: {wall_ms * 1e3:.1f} us/step wall, {kern_ms * 1e3:.1f} us/kernel (median "
        f"{np.median(kern) * 1e3:.1f}, min {kern.min() * 1e3:.1f}), {value:.1f} TFLOP/s")
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": p.dtype, "data": "synthetic (seeded numpy normal, RNE to bf16)",
        "config": {"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Lq": p.Lq, "Lk": p.Lk, "d": p.d,
                   "mask": p.mask_kind, "seed": p.meta.get("seed"), "flops_per_step": flops,
                   "plan": plan},
        "roofline": headline_roofline(args.only, p, plan, flops, kern, warm_ms),
        "parity": ("tests/test_gpu_parity.py::test_full_size_every_element compares every element of this "
                   "workload at this size against the oracle" if args.only in ("c3p", "c3d", "c5") else
                   "tests/test_gpu_parity.py::test_full_size_long_causal_16_heads compares 16 (batch, head) pairs of "
                   "this workload at this size against the oracle, every row" if args.only.startswith("c4") else
                   "tests/test_gpu_parity.py compares this workload against the oracle"),
    }
    del r
    torch.cuda.empty_cache()
    oracle_on = not args.no_cpu_baseline
    if not args.no_configs:
        configs = {}
        for key, label, run in config_entries(oracle_on):
            if wanted and key not in wanted:
                continue
            log(label)
            configs[key] = run()
        line["configs"] = configs
        if "c3d" in configs:
            d = configs["c3d"]
            rs = bench_read_stream(2 * d["B"] * d["Hkv"] * d["Lk"] * d["d"] * 2)
            line["decode"] = {"workload": d["workload"], "value": d["gbs"], "unit": "GB/s",
                              "frac_hbm_peak": round(d["gbs"] / PEAK_HBM_GBS, 4),
                              "read_stream": rs, "frac_of_read_stream": round(d["gbs"] / rs["best_gbs"], 4),
                              "roofline": {"bound": "hbm", "kernel": "decode_kernel<bf16,128> + lse_merge_kernel",
                                           "achieved": d["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                           "frac": round(d["gbs"] / PEAK_HBM_GBS, 4),
                                           "traffic": measured_traffic("decode_kernel<bf16,128,causal> c3 decode")}}
    if oracle_on:
        log("cpu baseline (fp64 oracle) on the headline workload")
        line["cpu_baseline"] = cpu_oracle(p, label=args.only)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
