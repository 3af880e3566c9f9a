"""fp64 CPU oracle for exact single-query attention decoding.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product library
(``long_context_attention_split_amd``) never imports, links or runs it, and this
package imports nothing from the product.

- ``decode_f64``: the plain definition softmax(q K^T d^-1/2 + bias) V, evaluated
  row by row in double precision by ``decode_f64.c`` (see its header for the
  formula and the pages it follows); fp32, bf16 and OCP fp8 (E4M3, E5M2) keys and
  values, fp8 with dequantisation scales per (batch, KV head) or per (batch, KV head,
  block of key positions).
- ``alibi_bias``: the bias term that definition adds ("ALiBi with causal=True
  unexpected bias?", causal bias vector example).
- ``tree``: numpy fp64 split-and-merge decoding (per-chunk peak / mass / value sum,
  then their combination), derived from the softmax over a union of key chunks that
  the tree-attention gist computes; used to pin the definition by chunk-count and
  merge-order invariance and to check per-chunk partials.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "decode_f64.c")
# ORACLE_LIB_PATH names another build of decode_f64.c (a host-sanitized one, say).
_OVERRIDE = os.environ.get("ORACLE_LIB_PATH")
_BUILT = os.path.join(_HERE, "liboracle_f64.so")
_LIB = _OVERRIDE or _BUILT
_lib = None

F32, BF16, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile decode_f64.c with gcc into liboracle_f64.so (host code only)."""
    if force or not os.path.exists(_BUILT) or os.path.getmtime(_BUILT) < os.path.getmtime(_SRC):
        tmp = _BUILT + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                               "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _BUILT)
    return _BUILT


def _load():
    global _lib
    if _lib is None:
        if not _OVERRIDE and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_decode_f64.restype = i32
        lib.oracle_decode_f64.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, i32, i64, i64, i64, i64, i64,
                                          i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, i64, i32, i64,
                                          vp, i32, vp, i32]
        lib.oracle_alibi_bias.restype = ctypes.c_double
        lib.oracle_alibi_bias.argtypes = [i64, i64, ctypes.c_double]
        lib.oracle_fp8_e4m3.restype = ctypes.c_double
        lib.oracle_fp8_e4m3.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_e5m2.restype = ctypes.c_double
        lib.oracle_fp8_e5m2.argtypes = [ctypes.c_uint8]
        _lib = lib
    return _lib


def _as_np(x):
    """numpy view of a CPU tensor/array; bf16 tensors become their uint16 bit patterns."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float8_e4m3fn:
                return x.view(torch.uint8).numpy(), FP8_E4M3
            if x.dtype == torch.float8_e5m2:
                return x.view(torch.uint8).numpy(), FP8_E5M2
            raise TypeError("oracle inputs must be fp32, bf16 or fp8, got %s" % x.dtype)
    except ImportError:
        pass
    x = np.asarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle inputs must be float32 or bf16 bits (uint16), got %s" % x.dtype)


def _strides(a: np.ndarray):
    es = a.itemsize
    if a.strides[-1] != es:
        raise ValueError("innermost dimension must be contiguous")
    return [s // es for s in a.strides]


def decode_f64(q, k, v, seq_lens=None, slopes=None, rows: Optional[Sequence[int]] = None,
               n_threads: Optional[int] = None, k_scale=None, v_scale=None, k_scale_block: int = 0,
               v_scale_block: int = 0) -> np.ndarray:
    """Oracle output (float64).

    q [B, Hq, d] or [B, Hq, nq, d] (nq query tokens, the last nq positions of each row,
    causal among themselves); k, v [B, Hkv, Lmax, d] (fp32, bf16 or fp8 torch tensors,
    or numpy float32 / uint16 bf16 bits); seq_lens int32 [B] or None; slopes fp32 [Hq]
    or None; k_scale, v_scale fp32 [B, Hkv] dequantisation scales (real = stored *
    scale) or None -- or, with k_scale_block / v_scale_block > 0, [B, Hkv, nblk]: key j
    uses block j // block.  ``rows``: flat (b*Hq+h)*nq+t indices to compute (result
    [len(rows), d]); None for all (result shaped like q).
    """
    lib = _load()
    qn, qt = _as_np(q)
    kn, kt = _as_np(k)
    vn, vt = _as_np(v)
    if kt != vt:
        raise TypeError("k and v must share a dtype")
    multi = qn.ndim == 4
    if not multi:
        qn = qn[:, :, None, :]
    B, Hq, nq, d = qn.shape
    Bk, Hkv, Lmax, dk = kn.shape
    if Bk != B or dk != d or vn.shape != kn.shape:
        raise ValueError("shape mismatch")
    sq, sk, sv = _strides(qn), _strides(kn), _strides(vn)
    sl = None
    if seq_lens is not None:
        sl = np.ascontiguousarray(np.asarray(seq_lens.cpu() if hasattr(seq_lens, "cpu") else seq_lens,
                                             dtype=np.int32))
    sp = None
    if slopes is not None:
        sp = np.ascontiguousarray(np.asarray(slopes.cpu() if hasattr(slopes, "cpu") else slopes,
                                             dtype=np.float32))
    def scales(x, block, name):
        if x is None:
            if block:
                raise ValueError("%s_scale_block given without %s_scale" % (name, name))
            return None, 0
        a = np.ascontiguousarray(np.asarray(x.cpu() if hasattr(x, "cpu") else x, dtype=np.float32))
        if block:
            if a.ndim != 3 or a.shape[:2] != (B, Hkv) or a.shape[2] * block < Lmax:
                raise ValueError("%s_scale must be [B, Hkv, >= ceil(Lmax / block)]" % name)
            return a.reshape(-1), a.shape[2]
        if a.size != B * Hkv:
            raise ValueError("%s_scale must hold B * Hkv values" % name)
        return a.reshape(-1), 0

    ksc, knb = scales(k_scale, k_scale_block, "k")
    vsc, vnb = scales(v_scale, v_scale_block, "v")
    rw = None
    n_rows = B * Hq * nq
    if rows is not None:
        rw = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        n_rows = int(rw.size)
    out = np.zeros((n_rows, d), dtype=np.float64)
    if n_threads is None:
        n_threads = len(os.sched_getaffinity(0))
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = lib.oracle_decode_f64(ptr(qn), qt, sq[0], sq[1], sq[2], nq, ptr(kn), ptr(vn), kt,
                               sk[0], sk[1], sk[2], sv[0], sv[1], sv[2],
                               B, Hq, Hkv, Lmax, d, ptr(sl), ptr(sp), ptr(ksc), ptr(vsc),
                               int(k_scale_block), int(knb), int(v_scale_block), int(vnb), ptr(rw), n_rows,
                               ptr(out), int(n_threads))
    if rc != 0:
        raise RuntimeError("oracle_decode_f64 failed (%d)" % rc)
    if rows is not None:
        return out
    return out.reshape(B, Hq, nq, d) if multi else out.reshape(B, Hq, d)


def alibi_bias(L: int, j: int, slope: float) -> float:
    """The bias the oracle adds to key j's scaled score for a sequence of length L."""
    return _load().oracle_alibi_bias(int(L), int(j), float(slope))


def fp8_value(bits: int, fmt: int) -> float:
    """The oracle's decoding of one FP8 byte (fmt FP8_E4M3 or FP8_E5M2)."""
    lib = _load()
    return lib.oracle_fp8_e4m3(bits) if fmt == FP8_E4M3 else lib.oracle_fp8_e5m2(bits)


def widen(x) -> np.ndarray:
    """Exact fp64 copy of an fp32 / bf16 / fp8 tensor (bf16: bits << 16; fp8: the
    oracle's own decoding table)."""
    a, t = _as_np(x)
    if t == F32:
        return a.astype(np.float64)
    if t in (FP8_E4M3, FP8_E5M2):
        table = np.array([fp8_value(i, t) for i in range(256)], dtype=np.float64)
        return table[a]
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
