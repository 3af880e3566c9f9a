"""GPU: tad_decode_noalloc, the entry point that takes no workspace and allocates nothing.

Its partials and counters live in the library's own device array, shared by every call
on a device.  Each call is checked against tad_decode_ws with the same n_splits (bit
for bit: the same kernels, the same chunking) and against the fp64 oracle, on calls in
a row whose sizes shrink, so that what an earlier call left in the array cannot leak
into a later one: a large grouped-query decode (matrix cores, split + combine), a d = 256
grouped-query decode (matrix cores at one wave per SIMD), then a one-head decode whose
chunks are cut into pieces (merged in the pieces kernel's last work-group: row
counters), then a small multi-head decode merged in the split kernel.
"""
import pytest
import torch

import oracle
import workloads as W
from test_parity_gpu import DEV, assert_parity, note, to_dev, vmax_real

pytestmark = pytest.mark.gpu


def run_pair(lib, c, S):
    g = to_dev(c)
    kw = dict(k_scale=g.get("k_scale"), v_scale=g.get("v_scale"))
    a = torch.full(g["q"].shape, float("nan"), dtype=torch.float32, device=DEV)
    lib.tad_decode_noalloc(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, a, **kw)
    torch.cuda.synchronize()
    b = torch.empty_like(a)
    ws = lib.workspace(g["q"], g["k"], lib.resolve_splits(g["q"], g["k"], S))
    lib.tad_decode_ws(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], lib.resolve_splits(g["q"], g["k"], S),
                      b, ws, **kw)
    torch.cuda.synchronize()
    return a, b


CASES = [
    ("grouped-query, 8 rows, ragged, automatic chunks", dict(seed=950, B=8, Hq=32, Hkv=8, L=6000, d=128,
                                                            seq_lens=[6000, 17, 0, 3001, 5999, 640, 1, 2048]), 0),
    ("d 256 grouped-query, 4 rows, ragged, automatic chunks", dict(seed=953, B=4, Hq=16, Hkv=4, L=3000, d=256,
                                                                   seq_lens=[3000, 1, 2999, 1500]), 0),
    ("one fp32 d=512 head, 8 chunks cut into pieces", dict(seed=951, B=1, Hq=1, Hkv=1, L=4096, d=512,
                                                          kv_dtype=torch.float32), 8),
    ("4 heads, 3 chunks, merged in the split kernel", dict(seed=952, B=1, Hq=4, Hkv=4, L=1000, d=64,
                                                         alibi=True), 3),
]


def test_noalloc_calls_in_a_row_shrinking(lib):
    for what, kw, S in CASES + CASES[::-1][1:]:     # large, smaller, smallest, then back up once
        note("noalloc: %s" % what)
        kw = dict(kw)
        c = W.random_case(kw.pop("seed"), kw.pop("B"), kw.pop("Hq"), kw.pop("Hkv"), kw.pop("L"), kw.pop("d"), **kw)
        a, b = run_pair(lib, c, S)
        assert torch.equal(a, b), what
        ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                                k_scale=c["k_scale"], v_scale=c["v_scale"])
        assert_parity(a.cpu().numpy(), ref, c["k"].dtype, vmax_real(c), what)


def test_noalloc_second_call_smaller_same_stream_no_sync(lib):
    """Two calls queued back to back on one stream, the second smaller, with no host
    synchronisation between them: stream order keeps them apart."""
    c1 = to_dev(W.random_case(960, 2, 16, 4, 5000, 128, seq_lens=[5000, 2222]))
    c2 = to_dev(W.random_case(961, 1, 2, 2, 700, 128))
    a1 = torch.empty(c1["q"].shape, dtype=torch.float32, device=DEV)
    a2 = torch.empty(c2["q"].shape, dtype=torch.float32, device=DEV)
    lib.tad_decode_noalloc(c1["q"], c1["k"], c1["v"], c1["seq_lens"], None, 0, a1)
    lib.tad_decode_noalloc(c2["q"], c2["k"], c2["v"], None, None, 2, a2)
    torch.cuda.synchronize()
    b1 = lib.decode(c1["q"], c1["k"], c1["v"], c1["seq_lens"], None, 0)
    b2 = lib.decode(c2["q"], c2["k"], c2["v"], None, None, 2)
    torch.cuda.synchronize()
    assert torch.equal(a1, b1) and torch.equal(a2, b2)


def test_noalloc_refuses_oversize_on_device(lib):
    """A call needing more partials than the array holds is refused, nothing runs, and
    a following call still works."""
    c = to_dev(W.random_case(970, 1, 128, 128, 200, 512, kv_dtype=torch.float32))   # ~26 MB of partials
    out = torch.zeros(c["q"].shape, dtype=torch.float32, device=DEV)
    with pytest.raises(lib.TadError) as e:
        lib.tad_decode_noalloc(c["q"], c["k"], c["v"], None, None, 100, out)
    assert e.value.code == lib.TAD_EWORKSPACE
    torch.cuda.synchronize()
    assert (out == 0).all()
    small = to_dev(W.random_case(971, 1, 2, 2, 300, 64))
    a = torch.empty(small["q"].shape, dtype=torch.float32, device=DEV)
    lib.tad_decode_noalloc(small["q"], small["k"], small["v"], None, None, 2, a)
    b = lib.decode(small["q"], small["k"], small["v"], None, None, 2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
