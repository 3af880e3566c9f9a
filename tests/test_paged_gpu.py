"""GPU parity of the paged K/V cache entry points against the fp64 oracle.

A contiguous seeded case is copied into a paged cache (workloads.page_kv: pages
handed out by a seeded permutation of the pool, unused rows NaN); the oracle runs on
the contiguous tensors, the GPU on the pages through tad_decode_paged_ws /
tad_decode_paged / tad_split_paged.  Same bars as the contiguous parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_parity_gpu import DEV, assert_parity, note, vmax_real

pytestmark = pytest.mark.gpu


def paged_case(seed, B, Hq, Hkv, L, d, ps, kv=torch.bfloat16, lens=None, alibi=False, nq=1,
               head_major=False):
    c = W.random_case(seed, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi)
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(seed + 9))
    kc, vc, table = W.page_kv(c["k"], c["v"], ps, seed, head_major=head_major)
    c.update(k_cache=kc, v_cache=vc, table=table)
    return c


def dev(x):
    return None if x is None else x.to(DEV)


def run_paged(lib, c, S, entry="ws"):
    q, kc, vc, tb = dev(c["q"]), dev(c["k_cache"]), dev(c["v_cache"]), dev(c["table"])
    sl, sp, ks, vs = dev(c["seq_lens"]), dev(c["slopes"]), dev(c.get("k_scale")), dev(c.get("v_scale"))
    if entry == "ws":
        out = lib.decode_paged(q, kc, vc, tb, sl, sp, S, k_scale=ks, v_scale=vs)
    else:
        out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        lib.tad_decode_paged(q, kc, vc, tb, sl, sp, S, out, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_of(c):
    return oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                             k_scale=c["k_scale"], v_scale=c["v_scale"])


@pytest.mark.parametrize("B,Hq,Hkv,L,d,ps,kv,S", [
    (2, 4, 4, 1000, 128, 16, torch.bfloat16, 5),           # MHA, vector path, fused merge
    (4, 32, 32, 1500, 128, 16, torch.bfloat16, 8),         # larger grid: split + combine
    (2, 16, 4, 1300, 128, 32, torch.bfloat16, 7),          # GQA 4: matrix-core path (one KV head per work-group)
    (2, 8, 4, 900, 64, 64, torch.bfloat16, 3),             # GQA 2, d 64, 64-row pages
    (2, 4, 2, 700, 256, 16, torch.bfloat16, 4),            # d 256, GQA 2: matrix cores (one wave per SIMD)
    (2, 4, 4, 1000, 128, 16, torch.float8_e4m3fn, 5),      # FP8 with scales, MHA
    (2, 8, 2, 1000, 128, 48, torch.float8_e5m2, 6),        # FP8 E5M2, GQA 4, 48-row pages
    (2, 4, 4, 600, 64, 16, torch.float8_e4m3fn, 3),        # FP8, d 64
    (1, 8, 8, 4096, 128, 256, torch.bfloat16, 0),          # 256-row pages, automatic splits
    (2, 32, 8, 1200, 128, 16, torch.float8_e4m3fn, 64),    # FP8 GQA, 4 KV heads per work-group (256 items)
    (3, 16, 4, 900, 128, 32, torch.float8_e5m2, 96),       # FP8 E5M2 GQA, 4 KV heads, split + combine
    (2, 32, 8, 1100, 64, 16, torch.bfloat16, 64),          # d 64 GQA, 4 KV heads per work-group
    (3, 16, 8, 1000, 64, 32, torch.float8_e4m3fn, 48),     # d 64 FP8 GQA, 4 KV heads, split + combine
    (2, 16, 4, 900, 64, 16, torch.float8_e5m2, 7),         # d 64 FP8: 32-key tiles over two 16-row pages, few items
    (2, 8, 2, 777, 128, 16, torch.float8_e4m3fn, 9),       # FP8, one KV head per work-group, 16-row pages
])
def test_paged_matches_oracle(lib, B, Hq, Hkv, L, d, ps, kv, S):
    """Ragged lengths (one not a page multiple) over a permuted page pool."""
    lens = [L, L * 2 // 3 + 5][:B] + [L // 3 + 1] * max(0, B - 2)
    note("paged B=%d Hq=%d Hkv=%d L=%d d=%d ps=%d kv=%s S=%d lens=%s" % (B, Hq, Hkv, L, d, ps, kv, S, lens))
    c = paged_case(600 + d + ps + B, B, Hq, Hkv, L, d, ps, kv, lens)
    ref = oracle_of(c)
    assert_parity(run_paged(lib, c, S), ref, kv, vmax_real(c), "paged")


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float8_e4m3fn])
@pytest.mark.parametrize("nq,Hkv", [(3, 2), (16, 8), (5, 4)])
def test_paged_several_tokens_alibi(lib, nq, Hkv, kv):
    """Several query tokens (causal among themselves) and ALiBi over a paged cache."""
    note("paged tokens nq=%d Hkv=%d kv=%s" % (nq, Hkv, kv))
    c = paged_case(650 + nq, 2, 8, Hkv, 800, 128, 16, kv, lens=[800, 333], alibi=True, nq=nq)
    ref = oracle_of(c)
    for S in (2, 9):
        out = run_paged(lib, c, S)
        assert out.shape == (2, 8, nq, 128)
        assert_parity(out, ref, kv, vmax_real(c), "paged tokens S=%d" % S)


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float8_e4m3fn])
@pytest.mark.parametrize("Hq", [4, 16])
def test_paged_head_major_pages(lib, kv, Hq):
    """Pages stored [Hkv, page_size, d] and described through strides."""
    note("paged head-major kv=%s Hq=%d" % (kv, Hq))
    c = paged_case(670 + Hq, 2, Hq, 4, 1000, 128, 32, kv, lens=[1000, 401], head_major=True)
    assert c["k_cache"].stride(2) == 32 * 128
    ref = oracle_of(c)
    assert_parity(run_paged(lib, c, 4), ref, kv, vmax_real(c), "head-major")


@pytest.mark.parametrize("ps,d,kv", [(16, 128, torch.bfloat16), (48, 128, torch.bfloat16), (32, 64, torch.bfloat16),
                                     (48, 256, torch.bfloat16), (16, 64, torch.float8_e4m3fn),
                                     (48, 128, torch.float8_e5m2), (16, 256, torch.float8_e4m3fn)])
def test_paged_head_major_tiles_across_pages(lib, ps, d, kv):
    """One query head per KV head on head-major pages (the vector kernel's paged form):
    its 32-key wave tiles are two 16-row pieces, each looked up in the block table on
    its own, so a tile may straddle two pages (16- and 48-row pages); ragged lengths
    that end inside a piece, an empty row, one and several chunks."""
    note("paged head-major tiles ps=%d d=%d kv=%s" % (ps, d, kv))
    c = paged_case(700 + ps + d, 3, 4, 4, 1000, d, ps, kv, lens=[1000, 333, 0], head_major=True)
    ref = oracle_of(c)
    for S in (1, 3, 0):
        out = run_paged(lib, c, S)
        assert_parity(out, ref, kv, vmax_real(c), "head-major tiles ps=%d S=%d" % (ps, S))
        assert (out[2] == 0).all()


def test_paged_entry_points_agree(lib):
    """tad_decode_paged (library workspace) equals tad_decode_paged_ws, and
    tad_split_paged + tad_combine equals both."""
    c = paged_case(680, 2, 16, 4, 1200, 128, 16, lens=[1200, 777])
    S = 6
    a = run_paged(lib, c, S, "ws")
    b = run_paged(lib, c, S, "alloc")
    assert np.array_equal(a, b)
    q, kc, vc, tb, sl = dev(c["q"]), dev(c["k_cache"]), dev(c["v_cache"]), dev(c["table"]), dev(c["seq_lens"])
    ws = torch.zeros(lib.tad_workspace_bytes(2, 16, 1, S, 128), dtype=torch.uint8, device=DEV)
    lib.tad_split_paged(q, kc, vc, tb, sl, None, S, ws)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lib.tad_combine(ws, 2, 16, 1, S, 128, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), a)


def test_paged_equals_contiguous_when_chunks_coincide(lib):
    """With a chunk length that is already a whole number of pages, the matrix-core
    kernel reads the same 16-key tiles in the same order from head-major pages as from
    the contiguous layout, so the paged and contiguous results are bit-identical."""
    c = paged_case(690, 2, 16, 4, 1024, 128, 16, lens=[1024, 1024], head_major=True)
    S = 4                                              # c = 256 keys = 16 pages
    a = run_paged(lib, c, S)
    g = {k: dev(c[k]) for k in ("q", "k", "v", "seq_lens")}
    b = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], None, S).cpu().numpy()
    assert np.array_equal(a, b)


def test_paged_unused_table_entries_are_not_read(lib):
    """Block-table entries past each row's length may hold anything; only the pages
    covering the first L_b keys are looked up."""
    c = paged_case(700, 2, 8, 2, 1000, 128, 16, lens=[1000, 300])
    table = c["table"].clone()
    table[1, 300 // 16 + 1:] = 1 << 30                 # far outside the pool
    c["table"] = table
    ref = oracle_of(c)
    assert_parity(run_paged(lib, c, 5), ref, torch.bfloat16, vmax_real(c), "unused entries")


def test_paged_out_of_range_pages_read_as_zeros(lib):
    """A block-table entry outside [0, num_pages) inside a row's length gives zero keys
    and values for that page (no fault); the oracle sees the same zeros."""
    c = paged_case(710, 2, 8, 2, 640, 128, 16, lens=[640, 500])
    n_pages = c["k_cache"].shape[0]
    table = c["table"].clone()
    table[0, 3] = n_pages + 7
    table[1, 10] = -5
    c["table"] = table
    k, v = c["k"].clone(), c["v"].clone()
    for b, p in ((0, 3), (1, 10)):
        k[b, :, p * 16:(p + 1) * 16] = 0
        v[b, :, p * 16:(p + 1) * 16] = 0
    ref = oracle.decode_f64(c["q"], k, v, seq_lens=c["seq_lens"])
    assert_parity(run_paged(lib, c, 4), ref, torch.bfloat16, vmax_real(c), "bad pages")
