"""GPU parity of grouped-query decode with more than 16 (head, token) columns per KV
head (query-head groups times query tokens, g * nq up to 256).

The matrix-core kernel cuts a KV head's g * nq columns into blocks of 16 (one product
width).  With per-(b, KV head) scales each wave runs two blocks on every tile it loads
(32 columns per read of the chunk); with FP8 block scales each block is a work-group of
its own.  A call with more blocks than a work-group takes gives each (chunk, group of
blocks) a work-group, those of one chunk on one XCD, one after another.  Every
case is held to the oracle's bars (fp64 definition: softmax over each token's visible
keys, times V), checked bit for bit against tad_split + tad_combine on a workspace
poisoned with NaN (a partial row no work-group wrote would surface), and repeated
(bit-identical calls).  The cases cover one and four KV heads per work-group, a last
group of fewer than 8 busy chunks, d 64 and 128, bf16, FP8 with per-head and per-block
scales, ALiBi, ragged rows shorter than nq, a paged cache, and 256 columns (16 blocks,
the most) next to 258 (the vector kernel).
"""
import random

import pytest
import torch

import oracle
import workloads as W
from test_block_scales_gpu import dequantised
from test_parity_gpu import DEV, assert_parity, note, to_dev, vmax_real, vmax_valid
from test_paged_gpu import paged_case, run_paged, oracle_of

pytestmark = pytest.mark.gpu

BF16, E4M3, E5M2 = torch.bfloat16, torch.float8_e4m3fn, torch.float8_e5m2


def tokens_case(seed, B, Hq, Hkv, nq, L, d, kv, lens, alibi, scale_block=0):
    c = W.random_case(seed, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi, scale_block=scale_block)
    c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(seed + 9))
    return c


def oracle_ref(c, blk=0):
    return oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                             k_scale=c["k_scale"], v_scale=c["v_scale"], k_scale_block=blk, v_scale_block=blk)


def vmax_of(c, blk):
    """max |V| over the valid keys, dequantised (per-head or per-block scales)."""
    if not blk:
        return vmax_real(c)
    v = dequantised(c["v"], c["v_scale"], blk)
    return vmax_valid(torch.from_numpy(v), c["seq_lens"])


def split_combine_poisoned(lib, g, S, blk):
    """tad_split into a workspace whose every byte is 0xFF (NaN partials; tad_split with
    several columns per KV head leaves the arrival counters alone), then tad_combine."""
    B, Hq, nq, d = g["q"].shape
    ws = lib.workspace(g["q"], g["k"], S)
    ws.fill_(0xFF)
    lib.tad_split(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, ws, k_scale=g.get("k_scale"),
                  v_scale=g.get("v_scale"), k_scale_block=blk, v_scale_block=blk)
    out = torch.empty((B, Hq, nq, d), dtype=torch.float32, device=DEV)
    lib.tad_combine(ws, B, Hq, nq, S, d, out)
    return out


@pytest.mark.parametrize("B,Hq,Hkv,nq,d,kv,lens,S,alibi,blk", [
    (2, 4, 4, 17, 128, BF16, [700, 15], 3, False, 0),        # 17 columns: 2 blocks, one KV head per WG
    (2, 8, 2, 5, 128, BF16, [900, 333], 5, True, 0),         # 4 heads x 5 tokens = 20
    (2, 8, 4, 9, 64, BF16, [1000, 7], 4, True, 0),           # 18 columns, d 64, a row shorter than nq
    (2, 32, 4, 4, 128, BF16, [1500, 1100], 4, False, 0),     # 8 heads x 4 tokens = 32, few items
    (2, 32, 4, 4, 128, BF16, [1500, 1100], 160, True, 0),    # 4 KV heads per WG; 125 busy chunks (8 q + 5)
    (3, 16, 1, 3, 64, E4M3, [800, 2, 1200], 6, False, 0),    # 16 heads x 3 tokens = 48, FP8 (2 WGs, one block empty)
    (2, 16, 4, 8, 128, E5M2, [1300, 640], 96, True, 64),     # 32 columns, 4 KV heads per WG, 64-key scale blocks (one block per WG)
    (1, 4, 2, 100, 64, BF16, [1000], 4, True, 0),            # 200 columns: 13 blocks
    (2, 64, 4, 16, 128, BF16, [640, 900], 7, False, 0),      # 256 columns: 16 blocks (the most)
    (1, 2, 1, 129, 64, BF16, [600], 3, False, 0),            # 258 columns: the vector kernel
])
def test_column_blocks_against_oracle(lib, B, Hq, Hkv, nq, d, kv, lens, S, alibi, blk):
    gq = Hq // Hkv * nq
    note("column blocks B=%d Hq=%d Hkv=%d nq=%d (g*nq=%d) d=%d kv=%s lens=%s S=%d alibi=%s blk=%d" %
         (B, Hq, Hkv, nq, gq, d, kv, lens, S, alibi, blk))
    c = tokens_case(900 + gq + d + S, B, Hq, Hkv, nq, max(lens), d, kv, lens, alibi, blk)
    ref = oracle_ref(c, blk)
    g = to_dev(c)
    a = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, k_scale=g.get("k_scale"),
                   v_scale=g.get("v_scale"), k_scale_block=blk, v_scale_block=blk)
    again = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, k_scale=g.get("k_scale"),
                       v_scale=g.get("v_scale"), k_scale_block=blk, v_scale_block=blk)
    b = split_combine_poisoned(lib, g, S, blk)
    torch.cuda.synchronize()
    assert torch.isfinite(b).all()
    assert torch.equal(a, again) and torch.equal(a, b)
    assert_parity(a.cpu().numpy(), ref, kv, vmax_of(c, blk), "column blocks g*nq=%d" % gq)
    for bb, L in enumerate(lens):
        if L < nq:                                   # tokens before the row's first key
            assert (a[bb, :, :nq - L] == 0).all()


@pytest.mark.parametrize("nq,ps,kv", [(6, 16, BF16), (12, 32, E4M3)])
def test_column_blocks_paged(lib, nq, ps, kv):
    """Paged cache (block table, 16- and 32-row pages), 4 query heads per KV head times
    nq tokens = 24 or 48 columns, ragged rows, ALiBi."""
    note("column blocks paged nq=%d ps=%d kv=%s" % (nq, ps, kv))
    c = paged_case(960 + nq, 2, 8, 2, 1100, 128, ps, kv, lens=[1100, 517], alibi=True, nq=nq)
    ref = oracle_of(c)
    for S in (5, 0):
        out = run_paged(lib, c, S)
        assert_parity(out, ref, kv, vmax_real(c), "paged column blocks S=%d" % S)


def draw_wide_cases(n, seed=2026):
    """Random calls with 17..256 (head, token) columns per KV head: batches across the
    64-row blocks of the work plan (70 rows), one to 8 KV heads, ragged lengths with
    zeros and rows shorter than nq, automatic and explicit chunk counts, ALiBi."""
    rnd = random.Random(seed)
    cases = []
    while len(cases) < n:
        d = rnd.choice([64, 128])
        kv = rnd.choice([BF16, BF16, E4M3, E5M2])
        Hkv = rnd.choice([1, 2, 4, 8])
        group = rnd.choice([1, 2, 4, 8, 16])
        nq = rnd.choice([2, 3, 4, 5, 8, 12, 16, 33])
        if not 16 < group * nq <= 256:
            continue
        B = rnd.choice([1, 2, 3, 8, 70])
        L = rnd.choice([17, 300, 1000, 2500, 6000])
        if B * Hkv * group * nq * L * d > 60_000_000:      # keep the oracle to a second or so
            L = max(nq + 1, 60_000_000 // (B * Hkv * group * nq * d))
        S = rnd.choice([0, 0, 1, 3, 8, 24, 100])
        cases.append((len(cases), B, Hkv * group, Hkv, nq, L, d, kv, B > 1 and rnd.random() < 0.8, S,
                      rnd.random() < 0.3))
    return cases


@pytest.mark.parametrize("case", draw_wide_cases(24), ids=lambda c: "w%d" % c[0])
def test_column_blocks_random(lib, case):
    i, B, Hq, Hkv, nq, L, d, kv, ragged, S, alibi = case
    lens = None
    if ragged:
        lens = torch.randint(0, L + 1, (B,), generator=torch.Generator().manual_seed(980 + i)).tolist()
        lens[0] = L
        lens[-1] = 0
        if B > 2:
            lens[1] = min(L, max(0, nq - 2))             # a row shorter than the tokens
    note("wide random %d: B=%d Hq=%d Hkv=%d nq=%d (g*nq=%d) L=%d d=%d kv=%s lens=%s S=%d alibi=%s" %
         (i, B, Hq, Hkv, nq, Hq // Hkv * nq, L, d, kv, "ragged" if ragged else "none", S, alibi))
    c = tokens_case(990 + i, B, Hq, Hkv, nq, L, d, kv, lens, alibi)
    ref = oracle_ref(c)
    g = to_dev(c)
    a = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, k_scale=g.get("k_scale"),
                   v_scale=g.get("v_scale"))
    SS = lib.resolve_splits(g["q"], g["k"], S)
    b = split_combine_poisoned(lib, g, SS, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "wide random case %d: decode differs from split + combine" % i
    assert_parity(a.cpu().numpy(), ref, kv, vmax_real(c), "wide random %d" % i)


@pytest.mark.parametrize("kv,d,nq", [(BF16, 128, 8), (E4M3, 64, 5), (BF16, 256, 3), (E5M2, 128, 2)])
def test_token_major_caches(lib, kv, d, nq):
    """K/V stored [B, L, Hkv, d] (the heads of a key next to each other), seen as
    [B, Hkv, L, d] through strides: 32 and 20 columns per KV head (two blocks per wave),
    d 256, and FP8 with 8 columns (4 KV heads per work-group from 256 items on, which
    such caches keep); small and large chunk counts."""
    from test_layouts_gpu import run_interleaved
    note("token-major kv=%s d=%d nq=%d" % (kv, d, nq))
    c = tokens_case(1400 + d + nq, 2, 16, 4, nq, 1500, d, kv, [1500, 777], True)
    ref = oracle_ref(c)
    for S in (5, 160):
        assert_parity(run_interleaved(lib, c, S), ref, kv, vmax_real(c), "token-major S=%d" % S)
