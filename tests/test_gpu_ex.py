"""GPU parity of attn_fwd_ex against the fp64 oracle (oracle/general.py): strided Q/K/V/out
(a transposed KV cache, padded rows), dense masks per batch and head with broadcast
strides, ALiBi and softcap, non-causal top-k and top-k with a dense mask, on the MFMA
prefill path (split and unsplit), the split-KV decode path and the fp32 row path."""
import numpy as np
import pytest

import synth
from helpers import compare, out_to_f64, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_flashattention_forward_amd as mfa
    mfa.lib()
    mfa.set_debug()
    yield
    mfa.set_debug()


def layout(t, kind):
    """The same values in another memory layout: 'bhld' contiguous, 'blhd' (heads inside
    rows, as a transposed cache), 'pad' (rows 16 elements apart beyond d)."""
    import torch
    if kind == "bhld":
        return t.contiguous()
    if kind == "blhd":
        return t.transpose(1, 2).contiguous().transpose(1, 2)
    if kind == "pad":
        B, H, L, d = t.shape
        buf = torch.full((B, H, L, d + 16), float("nan"), dtype=t.dtype, device=t.device)
        buf[..., :d] = t
        return buf[..., :d]
    if kind == "far":
        # rows FAR_ROW_STRIDE elements apart, NaN between them: a long cache slice whose
        # last row ends just under 2^31 bytes from its first
        B, H, L, d = t.shape
        buf = torch.full((B, H, L, FAR_ROW_STRIDE), float("nan"), dtype=t.dtype, device=t.device)
        buf[..., :d] = t
        return buf[..., :d]
    raise ValueError(kind)


FAR_ROW_STRIDE = 4096  # elements: 8 KB between 16-bit rows


def per_head_mask(seed, shape, Lq, Lk):
    rng = np.random.default_rng(seed)
    m = rng.standard_normal(shape + (Lq, Lk)).astype(np.float32)
    m[rng.random(m.shape) < 0.5] = -np.inf
    flat = m.reshape(-1, Lq, Lk)
    flat[0, min(1, Lq - 1)] = -np.inf         # a fully masked row in the first slice
    flat[-1, :, : Lk // 2] = -np.inf          # the last slice hides its first half
    return m


def run(p, *, qlay="bhld", klay="bhld", olay="bhld", mask=None, topk_causal=True, alibi=None, softcap=0.0,
        path=None, splits=0, heads=None):
    """attn_fwd_ex on device copies of p's stored inputs in the requested layouts, and
    the oracle on the same values."""
    import torch
    import masked_flashattention_forward_amd as mfa
    from oracle.general import general_attention_ref
    q = layout(to_device(p.q, p.dtype), qlay)
    k = layout(to_device(p.k, p.dtype), klay)
    v = layout(to_device(p.v, p.dtype), klay)
    out = layout(torch.full((p.B, p.Hq, p.Lq, p.d), float("nan"), dtype=q.dtype, device="cuda"), olay)
    lse = torch.full((p.B, p.Hq, p.Lq), float("nan"), dtype=torch.float32, device="cuda")
    zh = None if p.zero_hold is None else torch.from_numpy(p.zero_hold).cuda()
    md = None if mask is None else torch.from_numpy(mask).cuda()
    sl = None if alibi is None else torch.from_numpy(np.asarray(alibi, dtype=np.float32)).cuda()
    mfa.set_debug(force_path=-1 if path is None else path, force_splits=splits)
    try:
        mfa.attn_fwd_ex(q, k, v, scale=p.scale, mask_kind=p.mask_kind, window_left=p.window_left, mask=md,
                        zero_hold=zh, keep_k=p.keep_k, topk_causal=topk_causal, alibi_slopes=sl, softcap=softcap,
                        out=out, lse=lse)
        torch.cuda.synchronize()
    finally:
        mfa.set_debug()
    ref_o, ref_l = general_attention_ref(
        p.f64("q"), p.f64("k"), p.f64("v"), p.scale64, p.mask_kind, window_left=p.window_left,
        mask=None if mask is None else mask.astype(np.float64),
        zero_hold=None if p.zero_hold is None else p.zero_hold.astype(np.float64), keep_k=p.keep_k,
        topk_causal=topk_causal, alibi_slopes=None if alibi is None else np.asarray(alibi, dtype=np.float32),
        softcap=float(np.float32(softcap)), heads=heads)
    return out_to_f64(out, p.dtype), lse.cpu().numpy().astype(np.float64), ref_o, ref_l


def check(p, label, tol=None, **kw):
    say(label)
    out, lse, ref_o, ref_l = run(p, **kw)
    compare(p, out, lse, ref_o, ref_l, label=label, tol=tol)


# (dtype, d, Lq, Lk, Hq, Hkv, forced path, forced splits): prefill, split prefill, decode,
# and the fp32 row kernel
PATHS = [("bf16", 128, 77, 203, 4, 2, None, 0), ("fp16", 64, 77, 203, 4, 2, None, 0),
         ("bf16", 128, 77, 203, 4, 2, 1, 3), ("bf16", 128, 1, 1500, 8, 2, 2, 0), ("fp16", 64, 3, 900, 4, 1, 2, 0),
         ("fp32", 64, 33, 90, 4, 2, None, 0)]


def path_id(c):
    return f"{c[0]}-d{c[1]}-{c[2]}x{c[3]}-path{c[6]}-s{c[7]}"


@pytest.mark.parametrize("case", PATHS, ids=path_id)
@pytest.mark.parametrize("qlay,klay,olay", [("blhd", "blhd", "blhd"), ("bhld", "pad", "pad")])
@pytest.mark.parametrize("kind", ["causal", "dense", "topk"])
def test_strided_layouts(case, qlay, klay, olay, kind):
    dtype, d, Lq, Lk, Hq, Hkv, path, splits = case
    if kind == "topk" and path == 2 and Hq // Hkv * Lq > 32:
        pytest.skip("decode path rows")
    p = synth.make_problem(f"strided {kind}", 2, Hq, Hkv, Lq, Lk, d, dtype, kind, 900 + d + Lq,
                           keep_k=13, with_zero_hold=kind == "topk",
                           mask=per_head_mask(5, (), Lq, Lk) if kind == "dense" else None)
    check(p, f"strided {qlay}/{klay}/{olay} {kind} {path_id(case)}", qlay=qlay, klay=klay, olay=olay,
          mask=p.mask, path=path, splits=splits)


@pytest.mark.parametrize("case", PATHS, ids=path_id)
@pytest.mark.parametrize("varies", ["batch and head", "batch", "head", "neither"])
def test_per_head_dense_mask(case, varies):
    dtype, d, Lq, Lk, Hq, Hkv, path, splits = case
    shape = (2 if "batch" in varies else 1, Hq if "head" in varies else 1)
    m = per_head_mask(11 + shape[0] * 7 + shape[1], shape, Lq, Lk)
    p = synth.make_problem(f"per-head mask {shape}", 2, Hq, Hkv, Lq, Lk, d, dtype, "dense", 950 + d + Lq)
    check(p, f"dense mask varying with {varies} {path_id(case)}", mask=m, path=path, splits=splits)


SLOPES = {4: [0.5, 0.25, 0.125, 0.0625], 8: [2.0 ** -(i + 1) for i in range(8)]}


@pytest.mark.parametrize("case", PATHS, ids=path_id)
@pytest.mark.parametrize("kind", ["none", "causal", "window"])
@pytest.mark.parametrize("mods", ["alibi", "softcap", "both"])
def test_alibi_and_softcap(case, kind, mods):
    dtype, d, Lq, Lk, Hq, Hkv, path, splits = case
    # N(0,1) inputs (the absolute output bound assumes |v| of that size); a cap below the
    # logits' spread so that tanh bends them
    p = synth.make_problem(f"mods {kind}", 2, Hq, Hkv, Lq, Lk, d, dtype, kind, 1000 + d + Lq, window_left=41)
    alibi = SLOPES[Hq] if mods in ("alibi", "both") else None
    cap = 0.8 if mods in ("softcap", "both") else 0.0
    check(p, f"{mods} {kind} {path_id(case)}", alibi=alibi, softcap=cap, path=path, splits=splits)


def test_softcap_with_negative_scale():
    p = synth.make_problem("softcap negative scale", 1, 4, 2, 40, 130, 128, "bf16", "causal", 1100, scale=-0.09)
    check(p, p.name, softcap=1.7, alibi=SLOPES[4])


@pytest.mark.parametrize("dtype,d,Lq,Lk,Hq,Hkv,keep_k,path", [
    ("bf16", 128, 300, 1000, 2, 2, 40, None),   # kept-key lists (gathered tiles)
    ("fp16", 64, 77, 203, 4, 2, 150, None),    # every tile visited, per-tile minimum rank
    ("bf16", 128, 1, 2000, 8, 2, 100, 2),       # decode path
    ("fp32", 64, 20, 90, 2, 1, 30, None),       # row kernel
])
@pytest.mark.parametrize("with_mask", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_topk_variants(dtype, d, Lq, Lk, Hq, Hkv, keep_k, path, with_mask, causal):
    p = synth.make_problem("topk variants", 2, Hq, Hkv, Lq, Lk, d, dtype, "topk", 1200 + d + Lq, keep_k=keep_k,
                           with_zero_hold=True)
    m = per_head_mask(13, (2, Hq), Lq, Lk) if with_mask else None
    check(p, f"topk causal={causal} mask={with_mask} {dtype} d{d} {Lq}x{Lk} keep {keep_k} path {path}",
          mask=m, topk_causal=causal, path=path)


@pytest.mark.parametrize("kind", ["causal", "dense", "topk"])
def test_plain_call_matches_attn_fwd_bit_for_bit(kind):
    """Contiguous tensors and no modifier: attn_fwd_ex runs the same kernels as attn_fwd."""
    import torch
    import masked_flashattention_forward_amd as mfa
    p = synth.make_problem("ex vs fwd", 2, 8, 2, 130, 700, 128, "bf16", kind, 1300, keep_k=64,
                           with_zero_hold=kind == "topk", mask=per_head_mask(3, (), 130, 700) if kind == "dense" else None)
    say(p.name + " " + kind)
    q, k, v = (to_device(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    zh = None if p.zero_hold is None else torch.from_numpy(p.zero_hold).cuda()
    m = None if p.mask is None else torch.from_numpy(p.mask).cuda()
    o1, l1 = mfa.attn_fwd(q, k, v, scale=p.scale, mask_kind=kind, mask=m, zero_hold=zh, keep_k=p.keep_k)
    o2, l2 = mfa.attn_fwd_ex(q, k, v, scale=p.scale, mask_kind=kind, mask=m, zero_hold=zh, keep_k=p.keep_k)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.slow
@pytest.mark.parametrize("name", synth.EX_NAMES)
def test_ex_workloads_full_size_sampled(name):
    """The attn_fwd_ex workloads bench.py times, at their full size and in the same call,
    against the oracle on three sampled heads (all rows of each)."""
    p, o = synth.ex_config(name)
    heads = [(0, 0), (p.B // 2, p.Hq // 2 + 1), (p.B - 1, p.Hq - 1)]
    say(f"{name}: {p.name}")
    out, lse, ref_o, ref_l = run(p, qlay=o["layout"], klay=o["layout"], olay=o["layout"],
                                 mask=o["mask"] if o["mask"] is not None else p.mask, topk_causal=o["topk_causal"],
                                 alibi=o["alibi"], softcap=o["softcap"], heads=heads)
    compare(p, out, lse, ref_o, ref_l, heads=heads, label=f"{name} (sampled heads)")


@pytest.mark.parametrize("Lq,path,splits", [(1, None, 0), (16, None, 0), (16, 1, 1)])
def test_kv_slice_at_the_32bit_offset_limit(Lq, path, splits):
    """K and V slices whose last row ends just under 2^31 bytes from the first (262143 keys
    8 KB apart, NaN between the rows): the largest span the 32-bit offsets of the library
    take, on the decode path, the split prefill and one unsplit workgroup per query block
    (one key more is refused: tests/test_abi_cpu.py)."""
    Lk = 262143
    assert (Lk * FAR_ROW_STRIDE + 128) * 2 <= 2**31 - 1 < ((Lk + 1) * FAR_ROW_STRIDE + 128) * 2
    p = synth.make_problem(f"far rows Lq{Lq} Lk{Lk}", 1, 8, 1, Lq, Lk, 128, "bf16", "causal", 1701 + Lq)
    check(p, f"{p.name} path{path} splits{splits}", klay="far", path=path, splits=splits)


@pytest.mark.parametrize("Lk", [513, 2100])
@pytest.mark.parametrize("Lq,path", [(1, 2), (1, 1), (33, 1), (33, None)])
def test_mqa_per_head_mask_first_head_hidden(Lq, path, Lk):
    # One KV head and mask rows per query head, head 0 seeing no key at all: the dense-mask
    # tile summary must scan every query head of the group, not only the first (a tile
    # hidden from head 0 is still visible to the others). 2100 keys build the summary
    # flags on both paths, 513 keys visit every tile without them.
    Hq = 8
    m = per_head_mask(21 + Lq, (1, Hq), Lq, Lk)
    m[0, 0] = -np.inf
    p = synth.make_problem(f"MQA per-head mask Lq{Lq}", 1, Hq, 1, Lq, Lk, 128, "bf16", "dense", 970 + Lq)
    check(p, f"MQA per-head mask, head 0 hidden, Lq {Lq} path {path}", mask=m, path=path)
