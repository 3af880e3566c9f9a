"""GPU: one launch for small grouped-query decodes on the matrix cores.

When the matrix-core kernel serves one KV head per work-group, the call has at most 8
chunks and at most one (row, KV head, chunk) item per compute unit, tad_decode_ws
merges in the split kernel: the last of a (row, KV head) pair's non-empty chunks to
finish merges that KV head's g * nq (head, token) rows.  The result must equal
tad_split + tad_combine bit for bit (the merge keeps the combine's summation order),
stay within the parity bars of the fp64 oracle, leave the arrival counters at zero, and
give the same bits call after call through one workspace.
"""
import pytest
import torch

import oracle
import workloads as W
from test_parity_gpu import DEV, assert_parity, note, to_dev, vmax_real

pytestmark = pytest.mark.gpu


def counters_of(ws, rows, S, d):
    """The workspace's arrival counters (after m, l and o, each 256-byte aligned)."""
    al = lambda x: (x + 255) // 256 * 256
    n = rows * S
    off = 2 * al(4 * n) + al(4 * n * d)
    return ws[off:off + 4 * rows].view(torch.int32)


# (seed, B, Hq, Hkv, nq, L, d, kv, S, lens, alibi); S = 0: the automatic count
CASES = [
    (1, 1, 32, 8, 1, 4096, 128, torch.bfloat16, 8, None, False),      # one row, 64 work-groups
    (2, 1, 32, 8, 1, 4096, 128, torch.bfloat16, 4, None, False),
    (3, 3, 16, 4, 1, 5000, 128, torch.bfloat16, 8, [5000, 0, 1234], True),   # an empty row, ALiBi
    (4, 2, 16, 2, 1, 9000, 64, torch.float8_e4m3fn, 7, [9000, 3001], False),  # FP8 d 64, 8 heads per KV head
    (5, 2, 8, 2, 4, 3000, 128, torch.bfloat16, 8, [3000, 2], False),   # 4 tokens: 16 rows per merge
    (6, 4, 16, 4, 1, 20000, 128, torch.float8_e5m2, 8, None, False),  # 128 work-groups
    (7, 4, 8, 2, 2, 700, 128, torch.bfloat16, 5, [700, 1, 0, 64], True),  # tiny rows, one shorter than nq
    (8, 2, 8, 2, 1, 2000, 64, torch.bfloat16, 3, [0, 0], False),       # every row empty: zeros
    (9, 32, 8, 1, 1, 1500, 128, torch.bfloat16, 8, "random", False),   # 32 rows of one KV head, 256 work-groups
    (10, 1, 16, 1, 1, 3000, 64, torch.bfloat16, 2, None, True),        # 16 query heads on one KV head
    (11, 1, 16, 2, 1, 4096, 64, torch.bfloat16, 0, None, False),       # automatic chunk count
    (12, 100, 4, 1, 1, 300, 128, torch.bfloat16, 2, "random", True),   # more than 64 rows: the other plan path
    (13, 80, 8, 2, 1, 500, 64, torch.float8_e4m3fn, 1, "random", False),  # 80 rows, one chunk each
]


def fused_inputs(seed, B, Hq, Hkv, nq, L, d, kv, lens, alibi):
    if lens == "random":
        lens = torch.randint(0, L + 1, (B,), generator=torch.Generator().manual_seed(720 + seed)).tolist()
        lens[0], lens[1] = L, 0
    c = W.random_case(700 + seed, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi)
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(710 + seed))
    return c


@pytest.mark.parametrize("case", CASES, ids=lambda c: "f%d" % c[0])
def test_fused_grouped_decode_equals_split_combine(lib, case):
    seed, B, Hq, Hkv, nq, L, d, kv, S, lens, alibi = case
    note("fused mfma seed=%d B=%d Hq=%d Hkv=%d nq=%d L=%d d=%d kv=%s S=%d lens=%s alibi=%s" %
         (seed, B, Hq, Hkv, nq, L, d, kv, S, lens, alibi))
    c = fused_inputs(seed, B, Hq, Hkv, nq, L, d, kv, lens, alibi)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"])
    g = to_dev(c)
    kw = dict(k_scale=g.get("k_scale"), v_scale=g.get("v_scale"))
    shape = (B, Hq, nq, d) if nq > 1 else (B, Hq, d)
    S = lib.resolve_splits(g["q"], g["k"], S)
    ws = lib.workspace(g["q"], g["k"], S)
    outs = []
    for _ in range(3):                                 # one workspace, call after call
        o = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
        lib.tad_decode_ws(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, o, ws, **kw)
        outs.append(o)
    ws2 = lib.workspace(g["q"], g["k"], S)
    lib.tad_split(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, ws2, **kw)
    sc = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    lib.tad_combine(ws2, B, Hq, nq, S, d, sc)
    alloc = torch.empty(shape, dtype=torch.float32, device=DEV)
    lib.tad_decode(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], S, alloc, **kw)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, sc)
    assert torch.equal(alloc, sc)
    assert (counters_of(ws, B * Hq * nq, S, d) == 0).all()
    assert_parity(outs[0].cpu().numpy(), ref, kv, vmax_real(c), "fused mfma %d" % seed)
    for b in range(B):
        if c["seq_lens"] is not None and int(c["seq_lens"][b]) == 0:
            assert (outs[0][b] == 0).all()


def test_fused_grouped_decode_no_alloc_shrinking(lib):
    """The allocation-free entry point takes the same one-launch form: two calls in a
    row, the second smaller, each equal to tad_decode_ws."""
    for seed, B, L, S in ((30, 2, 6000, 8), (31, 1, 2500, 4)):
        c = to_dev(W.random_case(seed, B, 32, 8, L, 128, seq_lens=[L, L // 3][:B]))
        a = torch.empty((B, 32, 128), dtype=torch.float32, device=DEV)
        lib.tad_decode_noalloc(c["q"], c["k"], c["v"], c["seq_lens"], None, S, a)
        ws = lib.workspace(c["q"], c["k"], S)
        b = torch.empty_like(a)
        lib.tad_decode_ws(c["q"], c["k"], c["v"], c["seq_lens"], None, S, b, ws)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_fused_grouped_decode_paged(lib):
    """Token-major pages (the matrix-core kernel's paged form) with the merge fused."""
    B, Hq, Hkv, L, d, S, ps = 2, 32, 8, 3000, 128, 8, 16
    c = W.random_case(740, B, Hq, Hkv, L, d, seq_lens=[3000, 1111])
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"])
    kc, vc, table = W.page_kv(c["k"], c["v"], ps, 740)
    g = to_dev(c)
    kc, vc, table = kc.to(DEV), vc.to(DEV), table.to(DEV)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    ws = lib.workspace(g["q"], g["k"], S)
    lib.tad_decode_paged_ws(g["q"], kc, vc, table, g["seq_lens"], None, S, out, ws)
    ws2 = lib.workspace(g["q"], g["k"], S)
    lib.tad_split_paged(g["q"], kc, vc, table, g["seq_lens"], None, S, ws2)
    out2 = torch.empty_like(out)
    lib.tad_combine(ws2, B, Hq, 1, S, d, out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert_parity(out.cpu().numpy(), ref, torch.bfloat16, vmax_real(c), "fused mfma paged")
