"""GPU parity for K/V caches whose heads are interleaved per key.

A [B, L, Hkv, d] cache described as [B, Hkv, L, d] through strides (and paged caches
with [page_size, Hkv, d] pages) store the heads of one key next to each other; with
one query head per KV head the library reads them with the head-packed split kernel.
Checked against the fp64 oracle on the same values, at the usual bars, across
dtypes, head dims, chunk counts, ragged lengths and ALiBi; plus the fallbacks (head
counts the kernel cannot pack) and the agreement of the entry points.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_parity_gpu import DEV, assert_parity, note, vmax_real

pytestmark = pytest.mark.gpu


def interleave(x):
    """[B, H, L, d] -> the same values stored [B, L, H, d], viewed as [B, H, L, d] on the GPU."""
    return x.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)


def run_interleaved(lib, c, S):
    g = lambda key: None if c.get(key) is None else c[key].to(DEV)
    k, v = interleave(c["k"]), interleave(c["v"])
    assert k.stride(1) == k.shape[-1]
    out = lib.decode(c["q"].to(DEV), k, v, g("seq_lens"), g("slopes"), S, k_scale=g("k_scale"),
                     v_scale=g("v_scale"))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_of(c):
    return oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                             k_scale=c["k_scale"], v_scale=c["v_scale"])


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float32, torch.float8_e4m3fn, torch.float8_e5m2])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_interleaved_heads_dtypes_and_dims(lib, kv, d):
    """16 heads (packed by 4), ragged lengths, several chunks."""
    note("interleaved kv=%s d=%d" % (kv, d))
    c = W.random_case(800 + d, 2, 16, 16, 1000, d, kv_dtype=kv, seq_lens=[1000, 613])
    ref = oracle_of(c)
    for S in (1, 7):
        assert_parity(run_interleaved(lib, c, S), ref, kv, vmax_real(c), "interleaved S=%d" % S)


@pytest.mark.parametrize("S", [1, 2, 5, 33, 300])
def test_interleaved_split_counts_alibi(lib, S):
    """Chunk counts from one to more chunks than keys per chunk tile; ALiBi; a zero
    length and a length of one."""
    c = W.random_case(820, 4, 8, 8, 1500, 128, seq_lens=[1500, 0, 1, 999], alibi=True)
    note("interleaved alibi S=%d" % S)
    out = run_interleaved(lib, c, S)
    assert_parity(out, oracle_of(c), torch.bfloat16, vmax_real(c), "interleaved alibi S=%d" % S)
    assert (out[1] == 0).all()


def test_interleaved_many_ragged_rows(lib):
    """80 rows (more than a wave has lanes) with lengths from 0 up, interleaved heads."""
    g = torch.Generator().manual_seed(7)
    lens = torch.randint(0, 257, (80,), generator=g).tolist()
    lens[3] = 0
    c = W.random_case(825, 80, 4, 4, 256, 128, seq_lens=lens)
    assert_parity(run_interleaved(lib, c, 3), oracle_of(c), torch.bfloat16, vmax_real(c), "80 rows")


def test_interleaved_bf16_query_and_large_logits(lib):
    c = W.random_case(830, 2, 8, 8, 3000, 128, q_dtype=torch.bfloat16, k_scale=6.0)
    assert_parity(run_interleaved(lib, c, 6), oracle_of(c), torch.bfloat16, vmax_real(c), "bf16 q")


@pytest.mark.parametrize("B,Hq,Hkv,nq,S", [(2, 32, 8, 1, 5), (3, 16, 4, 1, 1), (2, 32, 8, 2, 7), (1, 8, 8, 1, 33),
                                          (2, 64, 16, 1, 4)])
@pytest.mark.parametrize("alibi", [False, True])
def test_interleaved_grouped_query_heads(lib, B, Hq, Hkv, nq, S, alibi):
    """Grouped-query heads over a [B, L, Hkv, d] cache with a KV-head count divisible by
    4, on calls with few (row, KV-head group, chunk) items: the matrix-core kernel then
    serves one KV head per work-group (4 adjacent ones from 256 items on, below)."""
    note("interleaved gqa B=%d Hq=%d Hkv=%d nq=%d S=%d alibi=%s" % (B, Hq, Hkv, nq, S, alibi))
    lens = [1300, 777, 5][:B]
    c = W.random_case(880 + Hkv + nq + S, B, Hq, Hkv, 1300, 128, seq_lens=lens, alibi=alibi)
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, 128), generator=torch.Generator().manual_seed(881))
    out = run_interleaved(lib, c, S)
    assert_parity(out, oracle_of(c), torch.bfloat16, vmax_real(c), "interleaved gqa S=%d" % S)


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float8_e4m3fn])
@pytest.mark.parametrize("B,Hq,Hkv,nq,S", [(2, 32, 8, 1, 5), (3, 16, 4, 2, 9), (2, 16, 8, 1, 16)])
def test_interleaved_grouped_query_heads_d64(lib, kv, B, Hq, Hkv, nq, S):
    """d = 64 grouped-query heads over a [B, L, Hkv, d] cache, few items (one KV head
    per work-group), ragged lengths, ALiBi, one and several tokens."""
    note("interleaved gqa d64 kv=%s B=%d Hq=%d Hkv=%d nq=%d S=%d" % (kv, B, Hq, Hkv, nq, S))
    c = W.random_case(960 + Hkv + nq + S, B, Hq, Hkv, 1250, 64, kv_dtype=kv, seq_lens=[1250, 701, 3][:B],
                      alibi=True)
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, 64), generator=torch.Generator().manual_seed(961))
    assert_parity(run_interleaved(lib, c, S), oracle_of(c), kv, vmax_real(c), "interleaved gqa d64 S=%d" % S)


@pytest.mark.parametrize("kv", [torch.float8_e4m3fn, torch.float8_e5m2])
@pytest.mark.parametrize("S", [3, 16])
def test_interleaved_fp8_grouped_query_heads(lib, kv, S):
    """FP8 K/V in a [B, L, Hkv, d] cache with grouped-query heads (one KV head per
    work-group at these item counts)."""
    note("interleaved fp8 gqa kv=%s S=%d" % (kv, S))
    c = W.random_case(890 + S, 2, 32, 8, 1400, 128, kv_dtype=kv, seq_lens=[1400, 611], alibi=True)
    assert_parity(run_interleaved(lib, c, S), oracle_of(c), kv, vmax_real(c), "interleaved fp8 gqa S=%d" % S)


@pytest.mark.parametrize("kv,d,nq,S", [(torch.bfloat16, 128, 1, 16), (torch.float8_e4m3fn, 128, 1, 24),
                                       (torch.bfloat16, 64, 2, 16), (torch.float8_e5m2, 64, 1, 20)])
def test_interleaved_four_heads_per_work_group(lib, kv, d, nq, S):
    """Enough (row, 4-KV-head group, chunk) items (8 rows x 2 groups x S >= 256) for the
    matrix-core kernel to serve 4 adjacent KV heads per work-group on a [B, L, Hkv, d]
    cache: ragged lengths with an empty row, ALiBi, one and two tokens."""
    note("interleaved 4 heads per work-group kv=%s d=%d nq=%d S=%d" % (kv, d, nq, S))
    lens = [1500, 0, 733, 1499, 1, 1024, 640, 1200]
    c = W.random_case(970 + d + nq + S, 8, 32, 8, 1500, d, kv_dtype=kv, seq_lens=lens, alibi=True)
    if nq > 1:
        c["q"] = torch.randn((8, 32, nq, d), generator=torch.Generator().manual_seed(971))
    assert_parity(run_interleaved(lib, c, S), oracle_of(c), kv, vmax_real(c), "interleaved 4 heads S=%d" % S)


@pytest.mark.parametrize("Hq,Hkv", [(6, 6), (2, 2), (8, 2)])
def test_interleaved_fallbacks(lib, Hq, Hkv):
    """Head counts the kernel cannot pack (6 and 2 heads: it packs heads by 4)
    and query-head groups take the other kernels; results are the same."""
    c = W.random_case(840 + Hq, 2, Hq, Hkv, 900, 128, seq_lens=[900, 450])
    assert_parity(run_interleaved(lib, c, 4), oracle_of(c), torch.bfloat16, vmax_real(c), "fallback")


def test_interleaved_entry_points_agree(lib):
    """tad_decode_ws (one launch on the small grid, split + combine on the large one),
    tad_decode and tad_split + tad_combine are bit-identical for interleaved caches."""
    for B, H, S in ((1, 4, 2), (2, 32, 16)):
        c = W.random_case(850 + B, B, H, H, 2000, 128, seq_lens=[2000, 1234][:B])
        q, sl = c["q"].to(DEV), c["seq_lens"].to(DEV)
        k, v = interleave(c["k"]), interleave(c["v"])
        a = lib.decode(q, k, v, sl, None, S)
        b = torch.empty_like(a)
        lib.tad_decode(q, k, v, sl, None, S, b)
        ws = lib.workspace(q, k, S)
        lib.tad_split(q, k, v, sl, None, S, ws)
        cc = torch.empty_like(a)
        lib.tad_combine(ws, B, H, 1, S, 128, cc)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(a, cc)


def test_interleaved_partials_match_contiguous(lib):
    """The per-chunk partials of the head-packed kernel describe the same chunk
    statistics as those of the contiguous layout (m equal up to rounding, l and o
    close), chunk by chunk."""
    c = W.random_case(860, 1, 8, 8, 2048, 128)
    q = c["q"].to(DEV)
    S = 4
    m1, l1, o1 = lib.split_partials(q, c["k"].to(DEV), c["v"].to(DEV), None, None, S)
    m2, l2, o2 = lib.split_partials(q, interleave(c["k"]), interleave(c["v"]), None, None, S)
    torch.cuda.synchronize()
    np.testing.assert_allclose(m2.cpu().numpy(), m1.cpu().numpy(), rtol=0, atol=1e-5)
    np.testing.assert_allclose(l2.cpu().numpy(), l1.cpu().numpy(), rtol=1e-5, atol=0)
    np.testing.assert_allclose(o2.cpu().numpy(), o1.cpu().numpy(), rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("kv,d", [(torch.bfloat16, 128), (torch.float8_e4m3fn, 128), (torch.bfloat16, 64),
                                  (torch.float8_e5m2, 256)])
def test_paged_interleaved_heads(lib, kv, d):
    """Paged caches with [page_size, Hkv, d] pages and enough heads to pack."""
    from test_paged_gpu import paged_case, run_paged
    note("paged interleaved kv=%s d=%d" % (kv, d))
    c = paged_case(870 + d, 2, 16, 16, 1100, d, 16, kv, lens=[1100, 555])
    ref = oracle_of(c)
    for S in (3, 12):
        assert_parity(run_paged(lib, c, S), ref, kv, vmax_real(c), "paged interleaved S=%d" % S)


def counters_of(ws, rows, S, d):
    """The workspace's arrival counters (after m, l and o, each 256-byte aligned)."""
    al = lambda x: (x + 255) // 256 * 256
    off = 2 * al(4 * rows * S) + al(4 * rows * S * d)
    return ws[off:off + 4 * rows].view(torch.int32)


@pytest.mark.parametrize("kv,d,B,H,L,S,lens,alibi", [
    (torch.bfloat16, 128, 1, 4, 3000, 1, None, False),               # one group of 4 heads, one chunk
    (torch.bfloat16, 128, 2, 16, 2500, 8, [2500, 0], True),          # an empty row, ALiBi, 8 chunks
    (torch.float8_e4m3fn, 128, 3, 8, 4000, 5, [4000, 17, 2222], False),
    (torch.float32, 64, 2, 8, 1500, 3, [1500, 1], False),             # fp32 d 64, a row of one key
    (torch.float8_e5m2, 256, 1, 12, 2048, 7, None, True),             # d 256, 3 groups
    (torch.bfloat16, 64, 4, 32, 1000, 8, [1000, 640, 0, 999], False),  # 256 work-groups
])
def test_interleaved_one_launch_equals_split_combine(lib, kv, d, B, H, L, S, lens, alibi):
    """Small grids on interleaved caches run the head-packed kernel with the merge in its
    last work-group per (row, 4-head group): bit-identical to tad_split + tad_combine,
    call after call through one workspace whose counters it leaves at zero, and within
    the bars of the oracle."""
    note("interleaved one launch kv=%s d=%d B=%d H=%d S=%d lens=%s" % (kv, d, B, H, S, lens))
    c = W.random_case(880 + d + S, B, H, H, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi)
    g = lambda key: None if c.get(key) is None else c[key].to(DEV)
    q, sl, sp = c["q"].to(DEV), g("seq_lens"), g("slopes")
    kw = dict(k_scale=g("k_scale"), v_scale=g("v_scale"))
    k, v = interleave(c["k"]), interleave(c["v"])
    ws = lib.workspace(q, k, S)
    outs = []
    for _ in range(3):
        o = torch.full((B, H, d), float("nan"), dtype=torch.float32, device=DEV)
        lib.tad_decode_ws(q, k, v, sl, sp, S, o, ws, **kw)
        outs.append(o)
    ws2 = lib.workspace(q, k, S)
    lib.tad_split(q, k, v, sl, sp, S, ws2, **kw)
    sc = torch.full((B, H, d), float("nan"), dtype=torch.float32, device=DEV)
    lib.tad_combine(ws2, B, H, 1, S, d, sc)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, sc)
    assert (counters_of(ws, B * H, S, d) == 0).all()
    out = outs[0].cpu().numpy()
    assert_parity(out, oracle_of(c), kv, vmax_real(c), "interleaved one launch")
    for b in range(B):
        if lens is not None and lens[b] == 0:
            assert (out[b] == 0).all()


def test_paged_interleaved_one_launch(lib):
    """Token-major pages with one query head per KV head on a small grid: one launch,
    equal to tad_split_paged + tad_combine bit for bit."""
    from test_paged_gpu import paged_case
    B, H, L, d, S, ps = 2, 16, 1100, 128, 4, 16
    c = paged_case(895, B, H, H, L, d, ps, torch.bfloat16, lens=[1100, 555])
    g = lambda key: None if c.get(key) is None else c[key].to(DEV)
    q, sl = c["q"].to(DEV), g("seq_lens")
    kc, vc, tb = c["k_cache"].to(DEV), c["v_cache"].to(DEV), c["table"].to(DEV)
    out = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    ws = lib.workspace(q, c["k"], S)
    lib.tad_decode_paged_ws(q, kc, vc, tb, sl, None, S, out, ws)
    ws2 = lib.workspace(q, c["k"], S)
    lib.tad_split_paged(q, kc, vc, tb, sl, None, S, ws2)
    out2 = torch.empty_like(out)
    lib.tad_combine(ws2, B, H, 1, S, d, out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert_parity(out.cpu().numpy(), oracle_of(c), torch.bfloat16, vmax_real(c), "paged interleaved one launch")
