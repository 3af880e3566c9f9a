"""Host-side checks of libtad's C ABI that need no GPU.

The library must load, export every function include/tad.h declares, and reject
bad arguments with the documented error codes before anything reaches the device.
Descriptors here carry fake (but aligned) device addresses: validation never
dereferences them, and every call below fails or returns before a launch.
"""
import ctypes
import os
import re

import pytest

import long_context_attention_split_amd as tad

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tad.h")

FAKE = 0x10000000   # 256-byte aligned stand-in address, never dereferenced


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tad_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function(lib):
    declared = header_functions()
    assert set(declared) == set(tad.EXPORTS)
    so = lib.load()
    for name in declared:
        assert hasattr(so, name), name


def test_version_matches_header(lib):
    m = re.search(r"#define TAD_VERSION (\d+)", open(HEADER).read())
    assert lib.tad_version() == int(m.group(1))


def test_workspace_bytes_layout(lib):
    # m and l: rows*S floats each, 256-aligned; o: rows*S*d floats; cnt: rows int32
    assert lib.tad_workspace_bytes(1, 32, 1, 32, 128) == 2 * 4096 + 1024 * 128 * 4 + 256
    assert lib.tad_workspace_bytes(8, 32, 1, 16, 128) == 2 * 16384 + 4096 * 128 * 4 + 1024
    assert lib.tad_workspace_bytes(1, 32, 4, 32, 128) == 2 * 16384 + 4096 * 128 * 4 + 512   # 4 tokens
    # fewer than 256 (row, chunk) pairs: after cnt, the partials of
    # Pmax = min(512 / pairs, 16384 / d, 64) pieces per chunk
    # one d = 512 head in 8 chunks: Pmax 32
    assert lib.tad_workspace_bytes(1, 1, 1, 8, 512) == (2 * 256 + 8 * 512 * 4 + 256 + 2 * 1024
                                                        + 8 * 32 * 512 * 4)
    # 32 heads in 4 chunks (128 pairs): Pmax 4
    assert lib.tad_workspace_bytes(1, 32, 1, 4, 128) == (2 * 512 + 128 * 128 * 4 + 256 + 2 * 2048
                                                         + 512 * 128 * 4)
    assert lib.tad_workspace_bytes(0, 1, 1, 1, 64) == 0
    assert lib.tad_workspace_bytes(1, 1, 1, 0, 64) == 0
    assert lib.tad_workspace_bytes(1, 1, 0, 1, 64) == 0


def desc(shape, dtype=tad.TAD_BF16, strides=None, addr=FAKE):
    t = tad.TadTensor()
    t.data = addr
    t.dtype = dtype
    t.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        t.shape[i] = s
        t.stride[i] = st
    return t


def good(B=2, Hq=8, Hkv=2, L=100, d=128):
    return dict(q=desc([B, Hq, d], tad.TAD_F32), k=desc([B, Hkv, L, d]), v=desc([B, Hkv, L, d]),
                out=desc([B, Hq, d], tad.TAD_F32))


def call_split(so, a, n_splits=4, ws=FAKE, ws_bytes=1 << 30):
    return so.tad_split(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]), None, None,
                        n_splits, ws, ws_bytes, None)


def call_decode_ws(so, a, n_splits=4, ws=FAKE, ws_bytes=1 << 30):
    return so.tad_decode_ws(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]), None, None,
                            n_splits, ctypes.byref(a["out"]), ws, ws_bytes, None)


@pytest.mark.parametrize("mutate,code", [
    (lambda a: a.update(q=desc([2, 8, 96], tad.TAD_F32), k=desc([2, 2, 100, 96]), v=desc([2, 2, 100, 96]),
                        out=desc([2, 8, 96], tad.TAD_F32)), tad.TAD_EUNSUPPORTED),
    (lambda a: a.update(q=desc([2, 6, 128], tad.TAD_F32), out=desc([2, 6, 128], tad.TAD_F32),
                        k=desc([2, 4, 100, 128]), v=desc([2, 4, 100, 128])), tad.TAD_EINVAL),   # 6 % 4
    (lambda a: a.update(k=desc([2, 2, 100, 128], tad.TAD_F32)), tad.TAD_EDTYPE),               # k f32, v bf16
    (lambda a: a.update(k=desc([2, 2, 100, 128], 7), v=desc([2, 2, 100, 128], 7)), tad.TAD_EDTYPE),
    (lambda a: a.update(q=desc([2, 8, 128], 5)), tad.TAD_EDTYPE),
    (lambda a: a.update(k=desc([2, 2, 100, 128], addr=FAKE + 8)), tad.TAD_ELAYOUT),            # misaligned
    (lambda a: a.update(k=desc([2, 2, 100, 128], strides=[25600, 12800, 128, 2])), tad.TAD_ELAYOUT),
    (lambda a: a.update(k=desc([2, 2, 100, 128], strides=[25604, 12800, 128, 1])), tad.TAD_ELAYOUT),
    (lambda a: a.update(q=desc([3, 8, 128], tad.TAD_F32)), tad.TAD_EINVAL),                    # batch
    (lambda a: a.update(v=desc([2, 2, 99, 128])), tad.TAD_EINVAL),                             # k/v shape
    (lambda a: a.update(q=desc([2, 8, 64], tad.TAD_F32)), tad.TAD_EINVAL),                     # head dim
    (lambda a: a.update(q=desc([2, 8, 0, 128], tad.TAD_F32)), tad.TAD_EINVAL),                 # no tokens
    (lambda a: a.update(q=desc([2, 8, 257, 128], tad.TAD_F32)), tad.TAD_EUNSUPPORTED),         # > 256 tokens
    (lambda a: a.update(k=desc([2, 2, 100, 128], addr=0)), tad.TAD_EINVAL),                    # null data
    (lambda a: a.update(k=desc([200, 128])), tad.TAD_EINVAL),                                  # 2-D k
])
def test_split_rejects_bad_arguments(lib, mutate, code):
    so = lib.load()
    a = good()
    mutate(a)
    assert call_split(so, a) == code
    assert lib.tad_last_error() != ""


def test_fp8_and_scale_rules(lib):
    """FP8 is accepted for k/v (with or without scales), not for q or out; a scale on a
    non-FP8 tensor is refused."""
    so = lib.load()
    a = good()
    a["k"] = desc([2, 2, 100, 128], tad.TAD_FP8_E4M3)
    a["v"] = desc([2, 2, 100, 128], tad.TAD_FP8_E4M3)
    a["k"].scale = FAKE
    a["v"].scale = FAKE
    assert call_split(so, a, ws_bytes=0) == tad.TAD_EWORKSPACE        # validated up to the workspace
    a["v"] = desc([2, 2, 100, 128], tad.TAD_FP8_E5M2)
    assert call_split(so, a) == tad.TAD_EDTYPE                        # k and v formats differ
    b = good()
    b["q"] = desc([2, 8, 128], tad.TAD_FP8_E4M3)
    assert call_split(so, b) == tad.TAD_EDTYPE
    c = good()
    c["k"].scale = FAKE
    assert call_split(so, c) == tad.TAD_EINVAL
    d = good()
    d["out"] = desc([2, 8, 128], tad.TAD_FP8_E4M3)
    assert call_decode_ws(so, d) == tad.TAD_EDTYPE
    # FP8 rows of 64 elements are 64 bytes: still 16-byte aligned
    e = good(d=64)
    e["k"] = desc([2, 2, 100, 64], tad.TAD_FP8_E5M2)
    e["v"] = desc([2, 2, 100, 64], tad.TAD_FP8_E5M2)
    e["q"] = desc([2, 8, 64], tad.TAD_F32)
    assert call_split(so, e, ws_bytes=0) == tad.TAD_EWORKSPACE


def test_block_scale_rules(lib):
    """scale_block: 0 (one scale per (b, KV head)) or a power of two from 16 to 65536,
    on FP8 tensors with a scale array only; K and V choose independently."""
    so = lib.load()

    def fp8(kb, vb):
        a = good()
        a["k"] = desc([2, 2, 100, 128], tad.TAD_FP8_E4M3)
        a["v"] = desc([2, 2, 100, 128], tad.TAD_FP8_E4M3)
        a["k"].scale, a["v"].scale = FAKE, FAKE
        a["k"].scale_block, a["v"].scale_block = kb, vb
        return a

    for kb, vb in ((16, 0), (0, 64), (65536, 256), (32, 32)):
        assert call_split(so, fp8(kb, vb), ws_bytes=0) == tad.TAD_EWORKSPACE   # validated up to the workspace
    for n in (8, 48, 100, 131072, -16):
        assert call_split(so, fp8(0, n)) == tad.TAD_EUNSUPPORTED
        assert "scale_block" in lib.tad_last_error()
    a = fp8(16, 0)
    a["k"].scale = None                                               # blocks without scales
    assert call_split(so, a) == tad.TAD_EINVAL
    b = good()
    b["v"].scale_block = 16                                           # bf16 values
    assert call_split(so, b) == tad.TAD_EINVAL


def test_split_rejects_bad_splits_and_workspace(lib):
    so = lib.load()
    a = good()
    assert call_split(so, a, n_splits=0) == tad.TAD_EINVAL
    assert call_split(so, a, n_splits=4097) == tad.TAD_EINVAL
    need = lib.tad_workspace_bytes(2, 8, 1, 4, 128)
    assert call_split(so, a, ws_bytes=need - 1) == tad.TAD_EWORKSPACE
    assert call_split(so, a, ws=FAKE + 16) == tad.TAD_EWORKSPACE
    assert call_split(so, a, ws=0) == tad.TAD_EWORKSPACE
    assert "workspace" in lib.tad_last_error()


def test_null_descriptors(lib):
    so = lib.load()
    a = good()
    rc = so.tad_split(None, ctypes.byref(a["k"]), ctypes.byref(a["v"]), None, None, 4, FAKE, 1 << 30, None)
    assert rc == tad.TAD_EINVAL
    rc = so.tad_decode_ws(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]), None, None, 4,
                          None, FAKE, 1 << 30, None)
    assert rc == tad.TAD_EINVAL


def test_decode_ws_checks_out(lib):
    so = lib.load()
    a = good()
    a["out"] = desc([2, 8, 128], tad.TAD_BF16)
    assert call_decode_ws(so, a) == tad.TAD_EDTYPE
    a["out"] = desc([2, 7, 128], tad.TAD_F32)
    assert call_decode_ws(so, a) == tad.TAD_EINVAL
    a["out"] = desc([2, 8, 128], tad.TAD_F32, strides=[1024, 128, 2])
    assert call_decode_ws(so, a) == tad.TAD_ELAYOUT
    # several query tokens: out must carry the same token count
    a["q"] = desc([2, 8, 3, 128], tad.TAD_F32)
    a["out"] = desc([2, 8, 128], tad.TAD_F32)
    assert call_decode_ws(so, a) == tad.TAD_EINVAL
    a["out"] = desc([2, 8, 3, 128], tad.TAD_F32)
    need = lib.tad_workspace_bytes(2, 8, 3, 4, 128)
    assert call_decode_ws(so, a, ws_bytes=need - 1) == tad.TAD_EWORKSPACE


def test_combine_validation(lib):
    so = lib.load()
    out = desc([2, 8, 128], tad.TAD_F32)
    assert so.tad_combine(FAKE, 1 << 30, 2, 8, 1, 4, 96, ctypes.byref(out), None) == tad.TAD_EUNSUPPORTED
    assert so.tad_combine(FAKE, 1 << 30, 2, 8, 1, 0, 128, ctypes.byref(out), None) == tad.TAD_EINVAL
    assert so.tad_combine(FAKE, 10, 2, 8, 1, 4, 128, ctypes.byref(out), None) == tad.TAD_EWORKSPACE
    assert so.tad_combine(FAKE, 1 << 30, 2, 9, 1, 4, 128, ctypes.byref(out), None) == tad.TAD_EINVAL
    assert so.tad_combine(FAKE, 1 << 30, 2, 8, 2, 4, 128, ctypes.byref(out), None) == tad.TAD_EINVAL
    assert so.tad_combine(FAKE, 1 << 30, 2, 8, 0, 4, 128, ctypes.byref(out), None) == tad.TAD_EINVAL


def test_empty_batch_is_a_no_op(lib):
    """B = 0 validates and returns success without touching the device."""
    so = lib.load()
    a = good(B=0)
    assert call_split(so, a) == tad.TAD_OK
    assert call_decode_ws(so, a) == tad.TAD_OK
    assert lib.tad_last_error() == ""


def test_chunk_span_limit(lib):
    """Chunks whose K rows would span >= 4 GiB are refused (32-bit buffer offsets)."""
    so = lib.load()
    L = 1 << 20
    a = good(B=1, Hq=1, Hkv=1, L=L)
    a["k"] = desc([1, 1, L, 128], strides=[L * 4096, L * 4096, 4096, 1])   # 8 KiB rows
    a["v"] = desc([1, 1, L, 128], strides=[L * 4096, L * 4096, 4096, 1])
    assert call_split(so, a, n_splits=1) == tad.TAD_EUNSUPPORTED
    assert call_split(so, a, n_splits=4, ws_bytes=0) == tad.TAD_EWORKSPACE   # passes the span check


def test_work_count_limit(lib):
    """Calls whose B * Hq * nq * n_splits exceeds 2^31 - 1 are refused before any launch
    (the kernels count work-groups in 32 bits); one under the limit passes that check."""
    so = lib.load()
    a = good(B=65536, Hq=64, Hkv=64, L=100)              # 2^22 rows
    assert call_split(so, a, n_splits=512) == tad.TAD_EUNSUPPORTED          # 2^31
    assert "exceeds" in lib.tad_last_error()
    assert call_split(so, a, n_splits=511, ws_bytes=0) == tad.TAD_EWORKSPACE  # passes the count check


def paged_good(B=2, Hq=8, Hkv=2, NP=20, PS=16, d=128, max_pages=7):
    return dict(q=desc([B, Hq, d], tad.TAD_F32), k=desc([NP, PS, Hkv, d]), v=desc([NP, PS, Hkv, d]),
                out=desc([B, Hq, d], tad.TAD_F32), pages=tad.TadPagedKv(FAKE, max_pages))


def call_split_paged(so, a, n_splits=4, ws=FAKE, ws_bytes=1 << 30, pages=True):
    pg = ctypes.byref(a["pages"]) if pages else None
    return so.tad_split_paged(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]), pg, None, None,
                              n_splits, ws, ws_bytes, None)


def call_decode_paged_ws(so, a, n_splits=4, ws=FAKE, ws_bytes=1 << 30):
    return so.tad_decode_paged_ws(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                                  ctypes.byref(a["pages"]), None, None, n_splits, ctypes.byref(a["out"]), ws,
                                  ws_bytes, None)


@pytest.mark.parametrize("mutate,code", [
    (lambda a: a.update(k=desc([20, 16, 2, 128], tad.TAD_F32), v=desc([20, 16, 2, 128], tad.TAD_F32)),
     tad.TAD_EDTYPE),                                                                        # fp32 cache
    (lambda a: a.update(k=desc([20, 24, 2, 128]), v=desc([20, 24, 2, 128])), tad.TAD_EUNSUPPORTED),  # page 24
    (lambda a: a.update(q=desc([2, 8, 512], tad.TAD_F32), k=desc([20, 16, 2, 512]), v=desc([20, 16, 2, 512]),
                        out=desc([2, 8, 512], tad.TAD_F32)), tad.TAD_EUNSUPPORTED),          # d 512
    (lambda a: a.update(k=desc([320, 2, 128])), tad.TAD_EINVAL),                             # 3-D cache
    (lambda a: a.update(v=desc([20, 16, 4, 128])), tad.TAD_EINVAL),                          # k/v heads differ
    (lambda a: a.update(v=desc([21, 16, 2, 128])), tad.TAD_EINVAL),                          # k/v pages differ
    (lambda a: a.update(k=desc([20, 16, 2, 128], strides=[4096, 256, 128, 2])), tad.TAD_ELAYOUT),
    (lambda a: a.update(k=desc([20, 16, 2, 128], strides=[4096, 256, 132, 1])), tad.TAD_ELAYOUT),  # 264 B
    (lambda a: a.update(k=desc([20, 16, 2, 128], strides=[4096, 100, 128, 1])), tad.TAD_ELAYOUT),  # overlap
    (lambda a: a.update(k=desc([20, 16, 2, 128], addr=FAKE + 8)), tad.TAD_ELAYOUT),
    (lambda a: a.update(pages=tad.TadPagedKv(FAKE, 0)), tad.TAD_EINVAL),                     # no pages
    (lambda a: a.update(pages=tad.TadPagedKv(None, 7)), tad.TAD_EINVAL),                     # null table
    (lambda a: a.update(pages=tad.TadPagedKv(FAKE, 1 << 27)), tad.TAD_EUNSUPPORTED),         # Lmax 2^31
    (lambda a: a.update(q=desc([2, 6, 128], tad.TAD_F32), k=desc([20, 16, 4, 128]), v=desc([20, 16, 4, 128])),
     tad.TAD_EINVAL),                                                                        # 6 % 4 heads
    (lambda a: a.update(q=desc([2, 8, 64], tad.TAD_F32)), tad.TAD_EINVAL),                   # head dim
])
def test_split_paged_rejects_bad_arguments(lib, mutate, code):
    so = lib.load()
    a = paged_good()
    mutate(a)
    rc = call_split_paged(so, a)
    assert rc == code, lib.tad_last_error()
    assert lib.tad_last_error() != ""


def test_paged_entry_points_validate_like_the_contiguous_ones(lib):
    so = lib.load()
    a = paged_good()
    assert call_split_paged(so, a, pages=False) == tad.TAD_EINVAL               # null pages descriptor
    assert call_split_paged(so, a, ws_bytes=0) == tad.TAD_EWORKSPACE           # all else valid
    assert call_split_paged(so, a, n_splits=0) == tad.TAD_EINVAL
    need = lib.tad_workspace_bytes(2, 8, 1, 4, 128)
    assert call_split_paged(so, a, ws_bytes=need - 1) == tad.TAD_EWORKSPACE
    # FP8 caches with scales are accepted; a scale on a bf16 cache is not
    f = paged_good()
    f["k"] = desc([20, 16, 2, 128], tad.TAD_FP8_E4M3)
    f["v"] = desc([20, 16, 2, 128], tad.TAD_FP8_E4M3)
    f["k"].scale = FAKE
    assert call_split_paged(so, f, ws_bytes=0) == tad.TAD_EWORKSPACE
    g = paged_good()
    g["k"].scale = FAKE
    assert call_split_paged(so, g) == tad.TAD_EINVAL
    # out is checked, several query tokens are accepted
    o = paged_good()
    o["out"] = desc([2, 8, 64], tad.TAD_F32)
    assert call_decode_paged_ws(so, o) == tad.TAD_EINVAL
    o["q"] = desc([2, 8, 5, 128], tad.TAD_F32)
    o["out"] = desc([2, 8, 5, 128], tad.TAD_F32)
    assert call_decode_paged_ws(so, o, ws_bytes=0) == tad.TAD_EWORKSPACE
    # a [num_pages, Hkv, page_size, d] cache seen through strides is a legal layout
    t = paged_good()
    t["k"] = desc([20, 16, 2, 128], strides=[4096, 128, 2048, 1])
    assert call_split_paged(so, t, ws_bytes=0) == tad.TAD_EWORKSPACE
    # empty batch: no-op success
    e = paged_good(B=0)
    assert call_split_paged(so, e) == tad.TAD_OK
    assert call_decode_paged_ws(so, e) == tad.TAD_OK
    rc = so.tad_decode_paged(ctypes.byref(e["q"]), ctypes.byref(e["k"]), ctypes.byref(e["v"]), None, None, None,
                             4, ctypes.byref(e["out"]), None)
    assert rc == tad.TAD_EINVAL


def test_auto_splits_without_device_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    so = lib.load()
    assert so.tad_auto_splits(1, 32, 32, 1, 131072, 128, tad.TAD_BF16, -1) == tad.TAD_EHIP
    assert so.tad_auto_splits(0, 32, 32, 1, 131072, 128, tad.TAD_BF16, -1) == tad.TAD_EINVAL
    assert so.tad_auto_splits(1, 12, 8, 1, 131072, 128, tad.TAD_BF16, -1) == tad.TAD_EINVAL   # Hq % Hkv
    assert so.tad_auto_splits(1, 32, 8, 0, 131072, 128, tad.TAD_BF16, -1) == tad.TAD_EINVAL   # nq
    assert so.tad_auto_splits(1, 32, 32, 1, 131072, 96, tad.TAD_BF16, -1) == tad.TAD_EUNSUPPORTED
    assert so.tad_auto_splits(1, 32, 32, 1, 131072, 128, 7, -1) == tad.TAD_EDTYPE


def test_product_does_not_reach_the_oracle():
    """The binding and the HIP sources never import, include or load the oracle."""
    pkg = os.path.join(ROOT, "long_context_attention_split_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_noalloc_refuses_calls_beyond_its_scratch(lib):
    """tad_decode_noalloc holds at most 16 MiB - 256 KiB of partials: a call needing more
    fails with TAD_EWORKSPACE before any device work (64 heads x 100 chunks x d 512 is
    about 26 MB of partials).  Bad arguments get the codes tad_decode gives."""
    so = lib.load()
    big = good(B=2, Hq=64, Hkv=64, L=1000, d=512)
    call = lambda a, S: so.tad_decode_noalloc(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                                              None, None, S, ctypes.byref(a["out"]), None)
    assert call(big, 100) == tad.TAD_EWORKSPACE
    assert "16" in lib.tad_last_error() or "scratch" in lib.tad_last_error()
    bad = good()
    bad["k"] = desc([2, 2, 100, 128], addr=0)
    assert call(bad, 4) == tad.TAD_EINVAL
    bad = good()
    bad["out"] = desc([2, 8, 128], tad.TAD_BF16)
    assert call(bad, 4) == tad.TAD_EDTYPE
    assert call(good(), 5000) == tad.TAD_EINVAL                         # n_splits beyond the maximum


def test_one_hip_runtime_in_the_process():
    """Loading the binding before anything else leaves one HIP runtime in the process
    (torch's, which libtad.so then shares), so torch tensors and streams are valid in
    the library."""
    import subprocess
    import sys
    code = ("import long_context_attention_split_amd as t; t.load(); "
            "m = open('/proc/self/maps').read().splitlines(); "
            "print('\\n'.join(sorted({l.split()[-1] for l in m if 'libamdhip64' in l})))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    paths = [p for p in out.stdout.split("\n") if p.strip()]
    assert len(paths) == 1, paths
