"""Python binding of libtad (split-KV exact attention decoding for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in ``include/tad.h``.  PyTorch supplies device memory and
streams.  The functions carry the C names:

- ``tad_decode(q, k, v, seq_lens, alibi_slopes, n_splits, out, stream=None)``
- ``tad_decode_noalloc(q, k, v, seq_lens, alibi_slopes, n_splits, out, stream=None)``
- ``tad_decode_ws(q, k, v, seq_lens, alibi_slopes, n_splits, out, ws, stream=None)``
- ``tad_split(q, k, v, seq_lens, alibi_slopes, n_splits, ws, stream=None)``
- ``tad_combine(ws, B, Hq, nq, n_splits, d, out, stream=None)``
- ``tad_auto_splits(B, Hq, Hkv, nq, Lmax, d, kv_dtype, device=-1)``, ``tad_workspace_bytes(B, Hq, nq, n_splits, d)``
- ``tad_workspace_clear(ws, stream=None)``, ``tad_version()``, ``tad_last_error()``
- ``tad_split_paged``, ``tad_decode_paged_ws``, ``tad_decode_paged``: the same with a
  paged K/V cache (k_cache, v_cache [num_pages, page_size, Hkv, d] and an int32
  block table [B, max_pages] in place of k and v)

and ``decode(...)`` allocates ``out`` and the workspace with torch and calls
``tad_decode_ws``.  Tensors: q [B, Hq, d] or [B, Hq, nq, d] (nq new tokens, causal)
fp32/bf16; k, v [B, Hkv, Lmax, d]
fp32/bf16/float8_e4m3fn/float8_e5m2 (innermost dim contiguous; FP8 with optional
k_scale / v_scale fp32 [B, Hkv], or [B, Hkv, nblk] with k_scale_block / v_scale_block
keys per scale block); seq_lens int32 [B] or None; alibi_slopes fp32
[Hq] or None; out fp32 shaped like q.  All must live on the GPU.

There is no fallback: if ``libtad.so`` has not been built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# TAD_LIB_PATH names another build of the same library (a host-sanitized one, say).
LIB_PATH = os.environ.get("TAD_LIB_PATH") or os.path.join(_HERE, "libtad.so")

TAD_F32, TAD_BF16, TAD_FP8_E4M3, TAD_FP8_E5M2 = 0, 1, 2, 3
TAD_OK, TAD_EINVAL, TAD_EDTYPE, TAD_ELAYOUT, TAD_EUNSUPPORTED, TAD_EWORKSPACE, TAD_EHIP = 0, -1, -2, -3, -4, -5, -6

EXPORTS = ("tad_version", "tad_last_error", "tad_auto_splits", "tad_workspace_bytes",
           "tad_workspace_clear", "tad_split", "tad_combine", "tad_decode_ws", "tad_decode",
           "tad_decode_noalloc", "tad_split_paged", "tad_decode_paged_ws", "tad_decode_paged")


class TadTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4), ("scale", ctypes.c_void_p),
                ("scale_block", ctypes.c_int32)]


class TadPagedKv(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32)]


class TadError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("libtad error %d: %s" % (code, msg))
        self.code = code


_lib = None


def load():
    """Load libtad.so (raises if it is missing: there is no CPU path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libtad.so is not built (%s); run __graft_entry__.build() or "
                           "python -m long_context_attention_split_amd.build" % LIB_PATH)
    # torch first: its HIP runtime is then the one libtad.so binds to (same soname), so
    # the process has one runtime and the tensors' device pointers and streams are
    # valid in the library.  Loaded first, the library would bring the system runtime
    # and torch would share that one instead of its own.
    _torch()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(TadTensor)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.tad_version.restype = ctypes.c_int
    lib.tad_version.argtypes = []
    lib.tad_last_error.restype = ctypes.c_char_p
    lib.tad_last_error.argtypes = []
    lib.tad_auto_splits.restype = i32
    lib.tad_auto_splits.argtypes = [i32, i32, i32, i32, i64, i32, i32, i32]
    lib.tad_workspace_bytes.restype = sz
    lib.tad_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.tad_workspace_clear.restype = ctypes.c_int
    lib.tad_workspace_clear.argtypes = [vp, sz, vp]
    lib.tad_split.restype = ctypes.c_int
    lib.tad_split.argtypes = [P, P, P, vp, vp, i32, vp, sz, vp]
    lib.tad_combine.restype = ctypes.c_int
    lib.tad_combine.argtypes = [vp, sz, i32, i32, i32, i32, i32, P, vp]
    lib.tad_decode_ws.restype = ctypes.c_int
    lib.tad_decode_ws.argtypes = [P, P, P, vp, vp, i32, P, vp, sz, vp]
    lib.tad_decode.restype = ctypes.c_int
    lib.tad_decode.argtypes = [P, P, P, vp, vp, i32, P, vp]
    lib.tad_decode_noalloc.restype = ctypes.c_int
    lib.tad_decode_noalloc.argtypes = [P, P, P, vp, vp, i32, P, vp]
    PG = ctypes.POINTER(TadPagedKv)
    lib.tad_split_paged.restype = ctypes.c_int
    lib.tad_split_paged.argtypes = [P, P, P, PG, vp, vp, i32, vp, sz, vp]
    lib.tad_decode_paged_ws.restype = ctypes.c_int
    lib.tad_decode_paged_ws.argtypes = [P, P, P, PG, vp, vp, i32, P, vp, sz, vp]
    lib.tad_decode_paged.restype = ctypes.c_int
    lib.tad_decode_paged.argtypes = [P, P, P, PG, vp, vp, i32, P, vp]
    _lib = lib
    return lib


# ----------------------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    """TAD_* code of a torch dtype (-1 for one the library does not take)."""
    torch = _torch()
    return {torch.float32: TAD_F32, torch.bfloat16: TAD_BF16, torch.float8_e4m3fn: TAD_FP8_E4M3,
            torch.float8_e5m2: TAD_FP8_E5M2}.get(dtype, -1)


def describe(t, scale=None, scale_block: int = 0) -> TadTensor:
    """tad_tensor for a torch tensor (no copy; the tensor must outlive the call's work).
    ``scale``: fp32 dequantisation scales of an FP8 k or v ([B, Hkv], or [B, Hkv, nblk]
    with ``scale_block`` keys per block), or None."""
    dt = dtype_code(t.dtype)
    if t.dim() > 4:
        raise ValueError("tensors have at most 4 dims")
    d = TadTensor()
    d.data = t.data_ptr() if t.numel() > 0 or t.data_ptr() else None
    d.dtype = dt
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    d.scale = None if scale is None else scale.data_ptr()
    d.scale_block = int(scale_block)
    return d


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> int:
    if rc != TAD_OK:
        raise TadError(rc, load().tad_last_error().decode())
    return rc


def tad_version() -> int:
    return load().tad_version()


def tad_last_error() -> str:
    return load().tad_last_error().decode()


def tad_auto_splits(B: int, Hq: int, Hkv: int, nq: int, Lmax: int, d: int, kv_dtype, device: int = -1) -> int:
    """kv_dtype: a TAD_* code or a torch dtype."""
    code = kv_dtype if isinstance(kv_dtype, int) else dtype_code(kv_dtype)
    r = load().tad_auto_splits(B, Hq, Hkv, nq, Lmax, d, code, device)
    if r < 0:
        _check(r)
    return r


def tad_workspace_bytes(B: int, Hq: int, nq: int, n_splits: int, d: int) -> int:
    return load().tad_workspace_bytes(B, Hq, nq, n_splits, d)


def tad_workspace_clear(ws, stream=None) -> int:
    return _check(load().tad_workspace_clear(ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def tad_split(q, k, v, seq_lens, alibi_slopes, n_splits: int, ws, stream=None, k_scale=None,
              v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0) -> int:
    lib = load()
    dq, dk, dv = describe(q), describe(k, k_scale, k_scale_block), describe(v, v_scale, v_scale_block)
    return _check(lib.tad_split(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _ptr(seq_lens),
                                _ptr(alibi_slopes), n_splits, ws.data_ptr(), ws.numel() * ws.element_size(),
                                _stream(stream)))


def tad_combine(ws, B: int, Hq: int, nq: int, n_splits: int, d: int, out, stream=None) -> int:
    lib = load()
    do = describe(out)
    return _check(lib.tad_combine(ws.data_ptr(), ws.numel() * ws.element_size(), B, Hq, nq, n_splits, d,
                                  ctypes.byref(do), _stream(stream)))


def tad_decode_ws(q, k, v, seq_lens, alibi_slopes, n_splits: int, out, ws, stream=None, k_scale=None,
                  v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0) -> int:
    lib = load()
    dq, do = describe(q), describe(out)
    dk, dv = describe(k, k_scale, k_scale_block), describe(v, v_scale, v_scale_block)
    return _check(lib.tad_decode_ws(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _ptr(seq_lens),
                                    _ptr(alibi_slopes), n_splits, ctypes.byref(do), ws.data_ptr(),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def tad_decode(q, k, v, seq_lens, alibi_slopes, n_splits: int, out, stream=None, k_scale=None,
               v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0) -> int:
    lib = load()
    dq, do = describe(q), describe(out)
    dk, dv = describe(k, k_scale, k_scale_block), describe(v, v_scale, v_scale_block)
    return _check(lib.tad_decode(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _ptr(seq_lens),
                                 _ptr(alibi_slopes), n_splits, ctypes.byref(do), _stream(stream)))


def tad_decode_noalloc(q, k, v, seq_lens, alibi_slopes, n_splits: int, out, stream=None, k_scale=None,
                       v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0) -> int:
    lib = load()
    dq, do = describe(q), describe(out)
    dk, dv = describe(k, k_scale, k_scale_block), describe(v, v_scale, v_scale_block)
    return _check(lib.tad_decode_noalloc(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _ptr(seq_lens),
                                         _ptr(alibi_slopes), n_splits, ctypes.byref(do), _stream(stream)))


def paged(block_table) -> TadPagedKv:
    """tad_paged_kv for an int32 [B, max_pages] device block table."""
    torch = _torch()
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [B, max_pages] tensor")
    p = TadPagedKv()
    p.block_table = block_table.data_ptr() if block_table.numel() else None
    p.max_pages = block_table.shape[1]
    return p


def tad_split_paged(q, k_cache, v_cache, block_table, seq_lens, alibi_slopes, n_splits: int, ws, stream=None,
                    k_scale=None, v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0) -> int:
    lib = load()
    dq, pg = describe(q), paged(block_table)
    dk, dv = describe(k_cache, k_scale, k_scale_block), describe(v_cache, v_scale, v_scale_block)
    return _check(lib.tad_split_paged(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(pg),
                                      _ptr(seq_lens), _ptr(alibi_slopes), n_splits, ws.data_ptr(),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def tad_decode_paged_ws(q, k_cache, v_cache, block_table, seq_lens, alibi_slopes, n_splits: int, out, ws,
                        stream=None, k_scale=None, v_scale=None, k_scale_block: int = 0,
                        v_scale_block: int = 0) -> int:
    lib = load()
    dq, do = describe(q), describe(out)
    dk, dv = describe(k_cache, k_scale, k_scale_block), describe(v_cache, v_scale, v_scale_block)
    pg = paged(block_table)
    return _check(lib.tad_decode_paged_ws(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(pg),
                                          _ptr(seq_lens), _ptr(alibi_slopes), n_splits, ctypes.byref(do),
                                          ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def tad_decode_paged(q, k_cache, v_cache, block_table, seq_lens, alibi_slopes, n_splits: int, out, stream=None,
                     k_scale=None, v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0) -> int:
    lib = load()
    dq, do = describe(q), describe(out)
    dk, dv = describe(k_cache, k_scale, k_scale_block), describe(v_cache, v_scale, v_scale_block)
    pg = paged(block_table)
    return _check(lib.tad_decode_paged(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(pg),
                                       _ptr(seq_lens), _ptr(alibi_slopes), n_splits, ctypes.byref(do),
                                       _stream(stream)))


def decode_paged(q, k_cache, v_cache, block_table, seq_lens=None, alibi_slopes=None, n_splits: int = 0,
                 stream=None, k_scale=None, v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0):
    """out = tad_decode_paged_ws(...) with torch-allocated out and workspace."""
    torch = _torch()
    B, Hq, d = q.shape[0], q.shape[1], q.shape[-1]
    Hkv, Lmax = k_cache.shape[2], block_table.shape[1] * k_cache.shape[1]
    S = n_splits if n_splits > 0 else tad_auto_splits(B, Hq, Hkv, tokens_of(q), Lmax, d, k_cache.dtype,
                                                      q.device.index or 0)
    nbytes = tad_workspace_bytes(B, Hq, tokens_of(q), S, d)
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    tad_decode_paged_ws(q, k_cache, v_cache, block_table, seq_lens, alibi_slopes, S, out, ws, stream,
                        k_scale, v_scale, k_scale_block, v_scale_block)
    return out


def shape_of(q, k):
    """(B, Hq, Hkv, Lmax, d) of a call's q and k."""
    B, Hq, d = q.shape[0], q.shape[1], q.shape[-1]
    if k.dim() == 4:
        Hkv, Lmax = k.shape[1], k.shape[2]
    else:
        Hkv, Lmax = 1, k.shape[1]
    return B, Hq, Hkv, Lmax, d


def resolve_splits(q, k, n_splits: int = 0) -> int:
    """n_splits if positive, else the library's automatic choice."""
    B, Hq, Hkv, Lmax, d = shape_of(q, k)
    return n_splits if n_splits > 0 else tad_auto_splits(B, Hq, Hkv, tokens_of(q), Lmax, d, k.dtype,
                                                         q.device.index or 0)


def tokens_of(q) -> int:
    """Query tokens per (b, h): 1 for [B, Hq, d], nq for [B, Hq, nq, d]."""
    return q.shape[2] if q.dim() == 4 else 1


def workspace(q, k, n_splits: int):
    """A zeroed torch-allocated workspace for (q, k) with n_splits chunks (uint8,
    256-aligned), ready for tad_decode_ws and reusable across calls."""
    torch = _torch()
    B, Hq, Hkv, Lmax, d = shape_of(q, k)
    nbytes = tad_workspace_bytes(B, Hq, tokens_of(q), n_splits, d)
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=q.device)


def decode(q, k, v, seq_lens=None, alibi_slopes=None, n_splits: int = 0, stream=None, k_scale=None,
           v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0):
    """out = tad_decode_ws(...) with torch-allocated out [B, Hq, d] fp32 and workspace."""
    torch = _torch()
    S = resolve_splits(q, k, n_splits)
    ws = workspace(q, k, S)
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    tad_decode_ws(q, k, v, seq_lens, alibi_slopes, S, out, ws, stream, k_scale, v_scale, k_scale_block,
                  v_scale_block)
    return out


def split_partials(q, k, v, seq_lens=None, alibi_slopes=None, n_splits: int = 1, stream=None,
                   k_scale=None, v_scale=None, k_scale_block: int = 0, v_scale_block: int = 0):
    """Run tad_split only; returns (m, l, o) views of the workspace:
    m, l [B, Hq, S] (m in base-2 units), o [B, Hq, S, d]."""
    torch = _torch()
    ws = workspace(q, k, n_splits)
    tad_split(q, k, v, seq_lens, alibi_slopes, n_splits, ws, stream, k_scale, v_scale, k_scale_block,
              v_scale_block)
    B, Hq, Hkv, Lmax, d = shape_of(q, k)
    nq = tokens_of(q)
    n = B * Hq * nq * n_splits
    al = lambda x: (x + 255) // 256 * 256
    off_l = al(4 * n)
    off_o = off_l + al(4 * n)
    lead = (B, Hq, nq) if q.dim() == 4 else (B, Hq)
    m = ws[0:4 * n].view(torch.float32).view(*lead, n_splits)
    l = ws[off_l:off_l + 4 * n].view(torch.float32).view(*lead, n_splits)
    o = ws[off_o:off_o + 4 * n * d].view(torch.float32).view(*lead, n_splits, d)
    return m, l, o
