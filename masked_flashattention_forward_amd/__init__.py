"""Masked FlashAttention forward for AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libmi_attn.so`` (declared in ``include/mi_attn.h``).
Torch tensors supply device memory and the stream; every step of the
computation runs in the library's HIP kernels. If the library has not been
built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmi_attn.so")

F32, F16, BF16 = 0, 1, 2
MASK_KINDS = {"none": 0, "causal": 1, "window": 2, "dense": 3, "topk": 4}
PATH_NAMES = {0: "row", 1: "mfma_prefill", 2: "splitkv_decode"}
OK, EINVAL, EUNSUPPORTED, EHIP = 0, -1, -2, -3


class MiAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mi_attn error {code}: {msg}")
        self.code = code


ABI_VERSION = 9  # MI_ATTN_ABI_VERSION of include/mi_attn.h that this binding matches


class AttnPlan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("splits", ctypes.c_int), ("grid", ctypes.c_int), ("mask_summary", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("topk_list_cap", ctypes.c_int)]


class AttnFwdArgs(ctypes.Structure):
    """attn_fwd_args_t of include/mi_attn.h (the same field order and types)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("lse", ctypes.c_void_p),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
                ("out_stride", ctypes.c_int64 * 3),
                ("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("Lq", ctypes.c_int),
                ("Lk", ctypes.c_int), ("d", ctypes.c_int), ("scale", ctypes.c_float), ("mask_kind", ctypes.c_int),
                ("window_left", ctypes.c_int), ("mask", ctypes.c_void_p), ("mask_stride", ctypes.c_int64 * 4),
                ("zero_hold", ctypes.c_void_p), ("keep_k", ctypes.c_int), ("topk_causal", ctypes.c_int),
                ("alibi_slopes", ctypes.c_void_p), ("softcap", ctypes.c_float), ("dtype", ctypes.c_int)]


_lib = None

_SIGS = {
    "attn_fwd": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int] * 6 + [ctypes.c_float]
                 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                    ctypes.c_void_p]),
    "attn_fwd_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int] * 6
                         + [ctypes.c_float] + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "dynamic_mask_topk": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_int] * 6
                          + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "attn_fwd_varlen": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_void_p, ctypes.c_int] * 2
                        + [ctypes.c_int] * 5 + [ctypes.c_float] + [ctypes.c_int] * 2
                        + [ctypes.c_void_p] + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3 + [ctypes.c_float]
                        + [ctypes.c_int, ctypes.c_void_p]),
    "attn_fwd_ex": (ctypes.c_int, [ctypes.POINTER(AttnFwdArgs), ctypes.c_void_p]),
    "attn_fwd_dump": (ctypes.c_int, [ctypes.POINTER(AttnFwdArgs)] + [ctypes.c_int] * 4
                      + [ctypes.c_void_p, ctypes.c_void_p]),
    "attn_bwd": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_void_p] * 4
                 + [ctypes.c_int] * 6 + [ctypes.c_float]
                 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                    ctypes.c_void_p]),
    "attn_fwd_plan": (ctypes.c_int, [ctypes.c_int] * 10 + [ctypes.POINTER(AttnPlan)]),
    "attn_set_debug": (None, [ctypes.c_int] * 3),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_abi_version": (ctypes.c_int, []),
    "attn_read_stream": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]),
}
EXPORTED = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch first: it ships its own HIP runtime under the same soname
        # (libamdhip64.so.7); loading the library before torch would bring the system
        # copy into the process as well, and two HIP runtimes do not share devices,
        # allocations or streams.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise MiAttnError(EHIP, f"{LIB_PATH} is missing: build it with "
                                    "`python -m masked_flashattention_forward_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        if l.attn_abi_version() != ABI_VERSION:
            raise MiAttnError(EHIP, f"{LIB_PATH} has ABI version {l.attn_abi_version()}, "
                                    f"this binding expects {ABI_VERSION}: rebuild it")
        _lib = l
    return _lib


def _check(rc: int):
    if rc != OK:
        raise MiAttnError(rc, lib().attn_last_error().decode())


def abi_version() -> int:
    return lib().attn_abi_version()


READ_STREAM_CHUNK = 2097152  # MI_ATTN_READ_STREAM_CHUNK
NOALLOC_MAX_WORKSPACE = 33554432  # MI_ATTN_NOALLOC_MAX_WORKSPACE
DUMP_FLOATS = 2 * 128 * 64 + 2 * 128  # MI_ATTN_DUMP_FLOATS


def read_stream(src, nontemporal: bool = True, sink=None, stream=None):
    """attn_read_stream: read every byte of the contiguous GPU tensor ``src`` once (a plain
    16-byte load stream; the measured HBM read ceiling for the decode roofline). Returns
    the int32 sink tensor the kernel writes (one word per 2 MiB)."""
    import torch
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    words = (nbytes + READ_STREAM_CHUNK - 1) // READ_STREAM_CHUNK
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=src.device)
    elif sink.numel() < words or sink.dtype != torch.int32:
        raise ValueError(f"sink must be int32 with at least {words} entries")
    if stream is None:
        stream = torch.cuda.current_stream(src.device)
    _check(lib().attn_read_stream(ctypes.c_void_p(src.data_ptr()), nbytes, int(bool(nontemporal)),
                                  ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream)))
    return sink


def set_debug(no_skip: bool = False, force_path: int = -1, force_splits: int = 0):
    lib().attn_set_debug(int(bool(no_skip)), int(force_path), int(force_splits))


_DTYPE_CODES = None  # torch dtype -> library dtype code, built on first use


def _dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def plan(B, Hq, Hkv, Lq, Lk, d, mask_kind="causal", window_left=0, keep_k=0, dtype=BF16) -> dict:
    """Which kernels attn_fwd runs for a shape (host-only)."""
    p = AttnPlan()
    mk = MASK_KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    _check(lib().attn_fwd_plan(B, Hq, Hkv, Lq, Lk, d, mk, window_left, keep_k, dtype, ctypes.byref(p)))
    return {"path": PATH_NAMES[p.path], "block_m": p.block_m, "block_n": p.block_n, "splits": p.splits,
            "grid": p.grid, "mask_summary": bool(p.mask_summary), "workspace_bytes": p.workspace_bytes,
            "topk_list_cap": p.topk_list_cap}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_raw_current_stream = None  # torch's accessor for the current stream's raw handle, looked up once


def _stream_handle(device, stream):
    """The HIP stream the call is enqueued on: ``stream`` (a torch stream), else torch's
    current stream of ``device``. The current stream's handle is read with torch's raw
    accessor, which skips building a stream object (about 1.8 us of host time per call)."""
    global _raw_current_stream
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    import torch
    if _raw_current_stream is None:
        _raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_current_stream and device.index is not None:
        return ctypes.c_void_p(_raw_current_stream(device.index))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def attn_fwd(q, k, v, *, scale=None, mask_kind="causal", window_left=0, mask=None, zero_hold=None,
             keep_k=0, out=None, lse=None, return_lse=True, stream=None, noalloc=False):
    """Masked attention forward (``noalloc=True``: attn_fwd_noalloc, the same call with its
    temporary memory taken from the library's fixed per-GPU scratch instead of allocated).

    q ``[B,Hq,Lq,d]``, k/v ``[B,Hkv,Lk,d]`` (fp32, fp16 or bf16, contiguous, on one
    GPU); mask ``[Lq,Lk]`` fp32 for ``mask_kind="dense"``; zero_hold ``[B,Hkv,Lk]``
    fp32 and ``keep_k`` for ``"topk"``. Returns ``(out, lse)``; lse is fp32
    ``[B,Hq,Lq]`` (natural log) or None when ``return_lse`` is false.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    B, Hq, Lq, d = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    mk = MASK_KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    if mask is not None:
        if mask.dtype != torch.float32 or tuple(mask.shape) != (Lq, Lk) or not mask.is_contiguous() \
                or mask.device != q.device:
            raise ValueError("mask must be a contiguous fp32 [Lq, Lk] tensor on q's device")
    if zero_hold is not None:
        if zero_hold.dtype != torch.float32 or tuple(zero_hold.shape) != (B, Hkv, Lk) \
                or not zero_hold.is_contiguous() or zero_hold.device != q.device:
            raise ValueError("zero_hold must be a contiguous fp32 [B, Hkv, Lk] tensor on q's device")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (B, Hq, Lq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [B, Hq, Lq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().attn_fwd_noalloc if noalloc else lib().attn_fwd
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Lq, Lk, d,
            float(scale), mk, int(window_left), _ptr(mask), _ptr(zero_hold), int(keep_k),
            _dtype_code(q), _stream_handle(q.device, stream))
    _check(rc)
    return out, lse


def attn_fwd_ex(q, k, v, *, scale=None, mask_kind="causal", window_left=0, mask=None, zero_hold=None, keep_k=0,
                topk_causal=True, alibi_slopes=None, softcap=0.0, out=None, lse=None, return_lse=True, stream=None,
                dump_at=None):
    """Masked attention forward with general layouts and score modifiers (attn_fwd_ex).

    q ``[B,Hq,Lq,d]`` and k/v ``[B,Hkv,Lk,d]`` may be any strided views whose last
    dimension is contiguous (a transposed cache ``[B,Lk,Hkv,d]`` passed as
    ``cache.transpose(1, 2)``). ``mask`` is an fp32 tensor that broadcasts to
    ``[B,Hq,Lq,Lk]`` (dense kind; with ``"topk"`` it is optional and added to the kept
    keys). ``topk_causal=False`` selects the top-k among all keys. ``alibi_slopes`` fp32
    ``[Hq]``; ``softcap`` > 0 caps the scaled scores. ``out`` may be strided too.
    Returns ``(out, lse)``. ``dump_at=(b, kv_head, query_block, tile)`` runs attn_fwd_dump
    instead and returns ``(out, lse, dump)`` with dump a dict of the tile's intermediates
    (``S``, ``P`` ``[128, 64]``, ``m``, ``l`` ``[128]``, NaN where not written).
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be a 4-D GPU tensor with a contiguous last dimension")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    B, Hq, Lq, d = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    mk = MASK_KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    mask_e = None
    if mask is not None:
        if mask.dtype != torch.float32 or mask.device != q.device:
            raise ValueError("mask must be an fp32 tensor on q's device")
        mask_e = mask.expand(B, Hq, Lq, Lk)  # broadcast dimensions get stride 0
    if zero_hold is not None:
        if zero_hold.dtype != torch.float32 or tuple(zero_hold.shape) != (B, Hkv, Lk) \
                or not zero_hold.is_contiguous() or zero_hold.device != q.device:
            raise ValueError("zero_hold must be a contiguous fp32 [B, Hkv, Lk] tensor on q's device")
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (Hq,) \
                or not alibi_slopes.is_contiguous() or alibi_slopes.device != q.device:
            raise ValueError("alibi_slopes must be a contiguous fp32 [Hq] tensor on q's device")
    if out is None:
        out = torch.empty((B, Hq, Lq, d), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (B, Hq, Lq, d) or out.dtype != q.dtype or out.stride(3) != 1:
        raise ValueError("out must match q's shape and dtype with a contiguous last dimension")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (B, Hq, Lq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [B, Hq, Lq] tensor")
    a = AttnFwdArgs()
    a.q, a.k, a.v, a.out = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = None if lse is None else lse.data_ptr()
    for dst, t in ((a.q_stride, q), (a.k_stride, k), (a.v_stride, v), (a.out_stride, out)):
        for i in range(3):
            dst[i] = t.stride(i)
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.d = B, Hq, Hkv, Lq, Lk, d
    a.scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    a.mask_kind, a.window_left = mk, int(window_left)
    if mask_e is not None:
        a.mask = mask_e.data_ptr()
        for i in range(4):
            a.mask_stride[i] = mask_e.stride(i)
    a.zero_hold = None if zero_hold is None else zero_hold.data_ptr()
    a.keep_k, a.topk_causal = int(keep_k), int(bool(topk_causal))
    a.alibi_slopes = None if alibi_slopes is None else alibi_slopes.data_ptr()
    a.softcap = float(softcap)
    a.dtype = _dtype_code(q)
    if dump_at is None:
        _check(lib().attn_fwd_ex(ctypes.byref(a), _stream_handle(q.device, stream)))
        return out, lse
    buf = torch.full((DUMP_FLOATS,), float("nan"), dtype=torch.float32, device=q.device)
    b, g, qb, tile = (int(x) for x in dump_at)
    _check(lib().attn_fwd_dump(ctypes.byref(a), b, g, qb, tile, ctypes.c_void_p(buf.data_ptr()),
                               _stream_handle(q.device, stream)))
    rows, keys = 128, 64
    dump = {"S": buf[:rows * keys].view(rows, keys), "P": buf[rows * keys:2 * rows * keys].view(rows, keys),
            "m": buf[2 * rows * keys:2 * rows * keys + rows], "l": buf[2 * rows * keys + rows:]}
    return out, lse, dump


def attn_bwd(q, k, v, out, lse, dout, *, scale=None, mask_kind="causal", window_left=0, mask=None, zero_hold=None,
             keep_k=0, dq=None, dk=None, dv=None, stream=None):
    """Gradients of attn_fwd: ``(dq, dk, dv)`` for the output gradient ``dout``.

    q, k, v, mask, zero_hold, keep_k and the mask arguments as given to attn_fwd; out and
    lse as it returned them (lse is required); dout like out. fp16/bf16, d 64 or 128.
    dq, dk and dv may be given (contiguous, shapes and dtype of q, k and v); they are
    overwritten.
    """
    import torch
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    for name, t, shape in (("q", q, (B, Hq, Lq, d)), ("k", k, (B, Hkv, Lk, d)), ("v", v, (B, Hkv, Lk, d)),
                           ("out", out, (B, Hq, Lq, d)), ("dout", dout, (B, Hq, Lq, d))):
        if not t.is_cuda or tuple(t.shape) != shape or not t.is_contiguous() or t.dtype != q.dtype \
                or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous {shape} {q.dtype} tensor on q's device")
    if lse is None or tuple(lse.shape) != (B, Hq, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be the contiguous fp32 [B, Hq, Lq] tensor attn_fwd wrote")
    mk = MASK_KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    if mask is not None:
        if mask.dtype != torch.float32 or tuple(mask.shape) != (Lq, Lk) or not mask.is_contiguous() \
                or mask.device != q.device:
            raise ValueError("mask must be a contiguous fp32 [Lq, Lk] tensor on q's device")
    if zero_hold is not None:
        if zero_hold.dtype != torch.float32 or tuple(zero_hold.shape) != (B, Hkv, Lk) \
                or not zero_hold.is_contiguous() or zero_hold.device != q.device:
            raise ValueError("zero_hold must be a contiguous fp32 [B, Hkv, Lk] tensor on q's device")
    grads = []
    for name, g, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if g is None:
            g = torch.empty_like(like)
        elif tuple(g.shape) != tuple(like.shape) or g.dtype != like.dtype or not g.is_contiguous():
            raise ValueError(f"{name} must match the shape and dtype of its input")
        grads.append(g)
    dq, dk, dv = grads
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rc = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                        B, Hq, Hkv, Lq, Lk, d, float(scale), mk, int(window_left),
                        _ptr(mask if mk == MASK_KINDS["dense"] else None),
                        _ptr(zero_hold if mk == MASK_KINDS["topk"] else None), int(keep_k), _dtype_code(q),
                        _stream_handle(q.device, stream))
    _check(rc)
    return dq, dk, dv


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, max_seqlen_q=None, max_seqlen_k=None,
                    block_table=None, k_new=None, v_new=None, scale=None, mask_kind="causal", window_left=0,
                    alibi_slopes=None, softcap=0.0, out=None, lse=None, return_lse=True, stream=None):
    """Masked attention over a batch of sequences of different lengths (attn_fwd_varlen).

    q ``[total_q, Hq, d]`` token-major; cu_seqlens_q/k int32 ``[num_seqs + 1]`` on q's
    device. With ``block_table`` (int32 ``[num_seqs, max_pages]``) k/v are a paged cache
    ``[num_pages, page_size, Hkv, d]``; without it they are packed ``[total_k, Hkv, d]``.
    ``k_new``/``v_new`` ``[total_q, Hkv, d]`` select the two-source form (the last Lq keys
    of each sequence). ``max_seqlen_q/k`` are host ints; when None they are read from the
    cu_seqlens tensors, which synchronises with the device. ``alibi_slopes`` fp32 ``[Hq]``
    and ``softcap`` as in attn_fwd_ex, on each sequence's own positions. Returns
    ``(out, lse)``, lse fp32 ``[total_q, Hq]``.
    """
    import torch

    def dev_tensor(name, t, dims, dtype=None):
        if not t.is_cuda or t.dim() != dims or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous {dims}-D tensor on q's device")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}")

    if not q.is_cuda or q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous 3-D GPU tensor [total_q, Hq, d]")
    total_q, Hq, d = q.shape
    paged = block_table is not None
    for name, t in (("k", k), ("v", v)):
        dev_tensor(name, t, 4 if paged else 3, q.dtype)
    if tuple(v.shape) != tuple(k.shape) or k.shape[-1] != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    Hkv = k.shape[-2]
    kv_rows = k.shape[0]
    page_size = k.shape[1] if paged else 0
    max_pages = 0
    if paged:
        dev_tensor("block_table", block_table, 2, torch.int32)
        max_pages = block_table.shape[1]
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        dev_tensor(name, t, 1, torch.int32)
    num_seqs = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != num_seqs + 1 or (paged and block_table.shape[0] != num_seqs):
        raise ValueError("cu_seqlens_q, cu_seqlens_k and block_table disagree on the number of sequences")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            dev_tensor(name, t, 3, q.dtype)
            if tuple(t.shape) != (total_q, Hkv, d):
                raise ValueError(f"{name} must be [total_q, Hkv, d]")
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if num_seqs else 0
    if max_seqlen_k is None:
        max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item()) if num_seqs else 0
    mk = MASK_KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (total_q, Hq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [total_q, Hq] tensor")
    if alibi_slopes is not None:
        dev_tensor("alibi_slopes", alibi_slopes, 1, torch.float32)
        if alibi_slopes.numel() != Hq:
            raise ValueError("alibi_slopes must be [Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rc = lib().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                               int(max_seqlen_q), _ptr(cu_seqlens_k), int(max_seqlen_k), num_seqs, total_q, Hq,
                               Hkv, d, float(scale), mk, int(window_left), _ptr(block_table), int(max_pages),
                               int(page_size), int(kv_rows), _ptr(k_new), _ptr(v_new), _ptr(alibi_slopes),
                               float(softcap), _dtype_code(q),
                               _stream_handle(q.device, stream))
    _check(rc)
    return out, lse


def dynamic_mask_topk(zero_hold, Lq, keep_k, causal=True, with_bits=False, stream=None):
    """Ranks ``[B,H,Lk]`` int32, thresholds ``[B,H,Lq]`` int32 and, if asked, the keep
    bitmask ``[B,H,Lq,ceil(Lk/32)]`` (as int32 words) of the dynamic top-k mask."""
    import torch
    if zero_hold.dtype != torch.float32 or zero_hold.dim() != 3 or not zero_hold.is_contiguous() \
            or not zero_hold.is_cuda:
        raise ValueError("zero_hold must be a contiguous fp32 [B, H, Lk] GPU tensor")
    B, H, Lk = zero_hold.shape
    dev = zero_hold.device
    rank = torch.empty((B, H, Lk), dtype=torch.int32, device=dev)
    tau = torch.empty((B, H, Lq), dtype=torch.int32, device=dev)
    bits = torch.empty((B, H, Lq, (Lk + 31) // 32), dtype=torch.int32, device=dev) if with_bits else None
    _check(lib().dynamic_mask_topk(_ptr(zero_hold), B, H, Lq, Lk, int(keep_k), int(bool(causal)),
                                   _ptr(rank), _ptr(tau), _ptr(bits), _stream_handle(dev, stream)))
    return rank, tau, bits
