"""GPU: chunks read by several work-groups ("pieces") and pre-merged inside the split
kernel, and the chunk-length rule of large grouped-query batches.

With few (row, chunk) pairs the vector kernel cuts every chunk into pieces, each read
by its own work-group; a second kernel merges the pieces' partials into the chunk's.  The chunks, and the partials tad_split reports, stay the ones n_splits asks
for: the partials must equal the oracle's per-chunk summaries at that chunk count,
tad_decode_ws must equal tad_split + tad_combine bit for bit, and the result must match
the fp64 oracle at the acceptance bars.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import tree
import workloads as W
from test_parity_gpu import DEV, assert_parity, note, to_dev, vmax_real

pytestmark = pytest.mark.gpu


def decode_both_ways(lib, g, S, out_shape, nq=1):
    """(tad_decode_ws output, tad_split + tad_combine output, the split's workspace)."""
    B, Hq, d = out_shape[0], out_shape[1], out_shape[-1]
    kw = dict(k_scale=g.get("k_scale"), v_scale=g.get("v_scale"))
    a = torch.empty(out_shape, dtype=torch.float32, device=DEV)
    ws = lib.workspace(g["q"], g["k"], S)
    lib.tad_decode_ws(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, a, ws, **kw)
    ws2 = lib.workspace(g["q"], g["k"], S)
    lib.tad_split(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, ws2, **kw)
    b = torch.empty_like(a)
    lib.tad_combine(ws2, B, Hq, nq, S, d, b)
    torch.cuda.synchronize()
    return a, b, ws2


@pytest.mark.parametrize("B,H,L,d,kv,S,lens,alibi", [
    (1, 1, 4096, 512, torch.float32, 8, None, False),         # one fp32 d = 512 head, 8 chunks
    (1, 1, 4096, 512, torch.float32, 3, None, True),          # ALiBi, chunks of 1366 keys
    (3, 2, 20000, 128, torch.bfloat16, 4, [20000, 7000, 0], False),   # ragged, an empty row
    (2, 4, 9000, 64, torch.bfloat16, 5, [9000, 4321], True),   # d = 64: 4 thread parts per column
    (1, 2, 30000, 256, torch.float8_e4m3fn, 2, None, False),  # FP8 with scales, d = 256
    (1, 1, 200000, 128, torch.bfloat16, 100, None, False),     # 100 chunks: pieces, then the combine kernel
])
def test_pieces_match_oracle_and_split_combine(lib, B, H, L, d, kv, S, lens, alibi):
    note("pieces B=%d H=%d L=%d d=%d kv=%s S=%d lens=%s alibi=%s" % (B, H, L, d, kv, S, lens, alibi))
    c = W.random_case(600 + d + S, B, H, H, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"])
    g = to_dev(c)
    a, b, _ = decode_both_ways(lib, g, S, (B, H, d))
    assert torch.equal(a, b)
    assert_parity(a.cpu().numpy(), ref, kv, vmax_real(c), "pieces S=%d" % S)


@pytest.mark.parametrize("lens", [None, [4096, 1500]])
def test_pieces_report_the_requested_chunks(lib, lens):
    """tad_split's partials are the summaries of the n_splits chunks the caller asked for
    (here 8 chunks of 512 keys, each read as several pieces), with m in base 2."""
    B, H, L, d, S = (1 if lens is None else 2), 1, 4096, 512, 8
    c = W.random_case(650 + (lens is not None), B, H, H, L, d, kv_dtype=torch.float32, seq_lens=lens)
    g = to_dev(c)
    m, l, o = lib.split_partials(g["q"], g["k"], g["v"], g["seq_lens"], None, S)
    torch.cuda.synchronize()
    m, l, o = m.cpu().double().numpy(), l.cpu().double().numpy(), o.cpu().double().numpy()
    clen = -(-L // S)
    for b in range(B):
        Lb = L if lens is None else lens[b]
        parts = tree.chunk_partials(oracle.widen(c["q"])[b, 0], oracle.widen(c["k"])[b, 0, :Lb],
                                    oracle.widen(c["v"])[b, 0, :Lb], S, None, clen)
        for s, (lm, den, num) in enumerate(parts):
            if den == 0.0:
                assert m[b, 0, s] == -np.inf and l[b, 0, s] == 0
                continue
            assert m[b, 0, s] * math.log(2) == pytest.approx(lm, rel=1e-5, abs=1e-5)
            fix = math.exp(m[b, 0, s] * math.log(2) - lm)
            assert l[b, 0, s] * fix == pytest.approx(den, rel=1e-4)
            np.testing.assert_allclose(o[b, 0, s] * fix, num, rtol=1e-4, atol=1e-4 * np.abs(num).max())


def test_pieces_paged_head_major(lib):
    """Pieces on a paged cache with head-major pages (the vector kernel's paged form):
    piece boundaries fall on whole pages."""
    B, H, L, d, S, ps = 2, 2, 5000, 128, 2, 16
    c = W.random_case(660, B, H, H, L, d, seq_lens=[5000, 3100])
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"])
    kc, vc, table = W.page_kv(c["k"], c["v"], ps, 660, head_major=True)
    g = to_dev(c)
    kc, vc, table = kc.to(DEV), vc.to(DEV), table.to(DEV)
    out = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    ws = lib.workspace(g["q"], g["k"], S)
    lib.tad_decode_paged_ws(g["q"], kc, vc, table, g["seq_lens"], None, S, out, ws)
    ws2 = lib.workspace(g["q"], g["k"], S)
    lib.tad_split_paged(g["q"], kc, vc, table, g["seq_lens"], None, S, ws2)
    out2 = torch.empty_like(out)
    lib.tad_combine(ws2, B, H, 1, S, d, out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert_parity(out.cpu().numpy(), ref, torch.bfloat16, vmax_real(c), "pieces paged")


def test_pieces_workspace_reused(lib):
    """One workspace reused for several calls with pieces keeps giving the same bits,
    and the fused merge's counter is left untouched at zero."""
    c = to_dev(W.random_case(670, 1, 1, 1, 4096, 512, kv_dtype=torch.float32))
    S, d = 8, 512
    ws = lib.workspace(c["q"], c["k"], S)
    outs = []
    for _ in range(4):
        out = torch.empty((1, 1, d), dtype=torch.float32, device=DEV)
        lib.tad_decode_ws(c["q"], c["k"], c["v"], None, None, S, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    al = lambda x: (x + 255) // 256 * 256
    n = 1 * S
    off_cnt = 2 * al(4 * n) + al(4 * n * d)
    counters = ws[off_cnt:off_cnt + 4].view(torch.int32)
    assert (counters == 0).all(), counters


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float8_e4m3fn])
def test_grouped_batch_beyond_resident_slots_keeps_its_chunks(lib, kv):
    """Matrix-core kernel with more (row, KV-head group) pairs than resident work-groups
    (72 rows x 4 groups of 4 KV heads = 288 > 256): the grid holds every item and the
    chunk length stays ceil(max L / n_splits), so the partials are those chunks."""
    B, Hq, Hkv, L, d, S = 72, 32, 16, 600, 128, 3
    gen = torch.Generator().manual_seed(680)
    lens = torch.randint(1, L + 1, (B,), generator=gen).tolist()
    lens[0], lens[5] = L, 0
    c = W.random_case(680 + (kv != torch.bfloat16), B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], k_scale=c["k_scale"],
                            v_scale=c["v_scale"])
    g = to_dev(c)
    a, b, ws = decode_both_ways(lib, g, S, (B, Hq, d))
    assert torch.equal(a, b)
    assert_parity(a.cpu().numpy(), ref, kv, vmax_real(c), "grouped beyond slots")
    m, l, o = lib.split_partials(g["q"], g["k"], g["v"], g["seq_lens"], None, S, k_scale=g["k_scale"],
                                 v_scale=g["v_scale"])
    torch.cuda.synchronize()
    m = m.cpu().numpy()
    clen = -(-max(lens) // S)
    for bb in range(B):
        busy = -(-lens[bb] // clen)
        assert np.isfinite(m[bb, :, :busy]).all(), bb
        assert np.isinf(m[bb, :, busy:]).all(), bb


def piece_cases(n=14, seed=4242):
    """Seeded random calls that cut their chunks into pieces: fewer than 256 (row, chunk)
    pairs, chunks of at least 256 KiB of K+V, any head dim and K/V dtype, ALiBi, ragged
    rows (a zero-length one included), one query row per KV head."""
    import random
    rnd = random.Random(seed)
    out = []
    for i in range(n):
        d = rnd.choice([64, 128, 256, 512])
        kv = rnd.choice([torch.float32, torch.bfloat16, torch.float8_e4m3fn, torch.float8_e5m2])
        if d == 512 and kv != torch.float32 and kv != torch.bfloat16:
            kv = torch.bfloat16
        elem = {torch.float32: 4, torch.bfloat16: 2}.get(kv, 1)
        B, H = rnd.choice([1, 2, 3]), rnd.choice([1, 2, 4])
        S = rnd.randint(1, max(1, 40 // (B * H)))
        keys = max(1, (256 << 10) // (2 * d * elem))          # one 256 KiB chunk
        L = S * keys * rnd.randint(1, 4) + rnd.randint(0, keys)
        L = min(L, 120000)
        lens = None
        if B > 1 and rnd.random() < 0.6:
            lens = [L] + [rnd.randint(0, L) for _ in range(B - 1)]
            if rnd.random() < 0.5:
                lens[-1] = 0
        out.append((i, B, H, L, d, kv, S, lens, rnd.random() < 0.4))
    return out


@pytest.mark.parametrize("case", piece_cases(), ids=lambda c: "c%d" % c[0])
def test_random_piece_cases(lib, case):
    i, B, H, L, d, kv, S, lens, alibi = case
    note("random pieces case %d: B=%d H=%d L=%d d=%d kv=%s S=%d lens=%s alibi=%s" % (i, B, H, L, d, kv, S, lens, alibi))
    c = W.random_case(700 + i, B, H, H, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"])
    g = to_dev(c)
    a, b, _ = decode_both_ways(lib, g, S, (B, H, d))
    assert torch.equal(a, b)
    # the allocating entry point cuts the call the same way
    e = torch.empty_like(a)
    lib.tad_decode(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, e, k_scale=g["k_scale"],
                   v_scale=g["v_scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, e)
    assert_parity(a.cpu().numpy(), ref, kv, vmax_real(c), "random pieces %d" % i)
