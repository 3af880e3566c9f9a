"""GPU: FP8 K/V with one dequantisation scale per block of key positions.

A tensor's ``scale_block`` = n gives key j of (b, KV head) the scale
scale[b, h, j // n] (a power of two n from 16 to 65536; K and V choose apart).  The
chunk length is rounded up to whole blocks, so every kernel's key tiles see one block
at a time.  Each case runs one kernel form -- the vector kernel (with pieces and
fused), the head-packed kernel, the matrix-core kernel (4 KV heads or 1 per
work-group, fused), each on a paged cache too -- and must match the fp64 oracle on
the dequantised values within the FP8 bar, and tad_decode_ws must equal tad_split +
tad_combine bit for bit.
"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import tree
from test_parity_gpu import DEV, assert_parity, note, vmax_valid

pytestmark = pytest.mark.gpu

E4, E5 = torch.float8_e4m3fn, torch.float8_e5m2


def dequantised(codes, scales, block):
    """fp64 values of FP8 codes [B, H, L, d] under block scales [B, H, >= ceil(L / block)]."""
    L = codes.shape[2]
    rep = np.repeat(scales.double().numpy(), block, axis=2)[:, :, :L]
    return np.nan_to_num(oracle.widen(codes)) * rep[:, :, :, None]


def block_case(seed, B, Hq, Hkv, nq, L, d, kv, lens, alibi, kb, vb):
    """Seeded inputs; K quantised in blocks of kb keys, V in blocks of vb keys."""
    c = W.random_case(seed, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi, scale_block=kb)
    v, vs = W.draw_kv_fp8_blocks(seed + 50, B, Hkv, L, d, vb, kv)
    if lens is not None:
        nan_bits = 0x7F if kv == E4 else 0x7E
        for b, Lb in enumerate(lens):
            v.view(torch.uint8)[b, :, Lb:, :] = nan_bits
    c["v"], c["v_scale"] = v, vs
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(seed + 9))
    return c


def padded(scales, block, Lcap):
    """Scales [B, H, n] widened to ceil(Lcap / block) blocks (a paged cache's logical
    length may exceed the drawn one); the extra blocks cover no key and hold 1."""
    n = -(-Lcap // block)
    out = torch.ones(scales.shape[0], scales.shape[1], n, dtype=torch.float32)
    out[:, :, :scales.shape[2]] = scales
    return out


# (seed, B, Hq, Hkv, nq, L, d, kv, S, lens, alibi, k block, v block, layout, kernel form)
CASES = [
    (1, 2, 4, 4, 1, 3000, 128, E4, 8, [3000, 1777], True, 16, 64, "contig", "vector"),
    (2, 1, 6, 6, 1, 5000, 64, E5, 0, None, False, 32, 32, "contig", "vector, automatic chunks"),
    (3, 1, 1, 1, 1, 20000, 256, E4, 4, None, False, 128, 256, "contig", "vector, pieces"),
    (4, 1, 2, 2, 1, 4096, 512, E4, 8, None, True, 16, 16, "contig", "vector d 512, pieces"),
    (5, 1, 4, 4, 1, 600, 128, E4, 4, None, False, 16, 32, "contig", "vector, one launch"),
    (6, 2, 4, 2, 1, 2500, 256, E5, 6, [2500, 999], False, 64, 16, "contig", "matrix cores, d 256"),
    (7, 1, 2, 2, 3, 1500, 512, E4, 5, None, False, 16, 16, "contig", "vector, 3 tokens"),
    (8, 2, 8, 8, 1, 4000, 128, E4, 8, [4000, 2100], True, 32, 128, "tokmajor", "head-packed"),
    (9, 1, 8, 8, 1, 1200, 64, E5, 4, None, False, 16, 16, "tokmajor", "head-packed, one launch"),
    (10, 8, 32, 8, 1, 6000, 128, E4, 24, "random", False, 64, 16, "contig", "matrix cores, 4 KV heads/WG"),
    (11, 2, 16, 4, 4, 3000, 64, E5, 8, [3000, 1500], True, 32, 32, "contig", "matrix cores, 4 tokens"),
    (12, 1, 32, 8, 1, 4096, 128, E4, 8, None, False, 16, 64, "contig", "matrix cores, one launch"),
    (13, 4, 16, 2, 1, 8000, 128, E4, 0, None, False, 256, 256, "contig", "matrix cores, automatic chunks"),
    (14, 2, 32, 8, 1, 3000, 128, E4, 8, [3000, 1111], False, 64, 32, "paged16", "matrix cores, paged"),
    (15, 2, 8, 8, 1, 2500, 64, E5, 6, [2500, 801], True, 16, 128, "paged32", "head-packed, paged"),
    (16, 2, 2, 2, 1, 2000, 128, E4, 5, [2000, 1300], False, 64, 64, "paged16hm", "vector, paged"),
    (17, 2, 8, 2, 1, 2000, 128, E4, 6, [2000, 700], False, 64, 16, "paged48", "matrix cores, 48-row pages"),
    (18, 1, 2, 2, 1, 20000, 128, E5, 2, None, False, 64, 128, "paged16hm", "vector, paged, pieces"),
    (19, 2, 4, 2, 1, 2500, 512, E5, 6, [2500, 999], False, 64, 16, "contig", "vector, query-head groups"),
]


def run_layout(lib, c, layout, S, kb, vb, entry):
    """One call through `entry` ("ws": tad_decode_ws, "alloc": tad_decode, "split":
    tad_split + tad_combine) on the case's layout; returns out on the GPU."""
    q = c["q"].to(DEV)
    dev = lambda key: None if c.get(key) is None else c[key].to(DEV)
    shape = q.shape
    out = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    B, Hq, d = q.shape[0], q.shape[1], q.shape[-1]
    nq = q.shape[2] if q.dim() == 4 else 1
    kw = dict(k_scale_block=kb, v_scale_block=vb)
    if layout.startswith("paged"):
        ps = int(layout[5:7])
        kc, vc, table = W.page_kv(c["k"], c["v"], ps, 900 + S, head_major=layout.endswith("hm"))
        Lcap = table.shape[1] * ps
        ks, vs = padded(c["k_scale"], kb, Lcap).to(DEV), padded(c["v_scale"], vb, Lcap).to(DEV)
        kc, vc, table = kc.to(DEV), vc.to(DEV), table.to(DEV)
        ws = lib.workspace(q, c["k"].to(DEV), S)
        args = (q, kc, vc, table, dev("seq_lens"), dev("slopes"), S)
        if entry == "ws":
            lib.tad_decode_paged_ws(*args, out, ws, k_scale=ks, v_scale=vs, **kw)
        elif entry == "alloc":
            lib.tad_decode_paged(*args, out, k_scale=ks, v_scale=vs, **kw)
        else:
            lib.tad_split_paged(*args, ws, k_scale=ks, v_scale=vs, **kw)
            lib.tad_combine(ws, B, Hq, nq, S, d, out)
        return out
    if layout == "tokmajor":
        k = c["k"].transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
        v = c["v"].transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
        assert k.stride(1) == d
    else:
        k, v = c["k"].to(DEV), c["v"].to(DEV)
    ks, vs = dev("k_scale"), dev("v_scale")
    ws = lib.workspace(q, k, S)
    args = (q, k, v, dev("seq_lens"), dev("slopes"), S)
    if entry == "ws":
        lib.tad_decode_ws(*args, out, ws, k_scale=ks, v_scale=vs, **kw)
    elif entry == "alloc":
        lib.tad_decode(*args, out, k_scale=ks, v_scale=vs, **kw)
    else:
        lib.tad_split(*args, ws, k_scale=ks, v_scale=vs, **kw)
        lib.tad_combine(ws, B, Hq, nq, S, d, out)
    return out


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d" % c[0])
def test_block_scaled_fp8_decode(lib, case):
    seed, B, Hq, Hkv, nq, L, d, kv, S, lens, alibi, kb, vb, layout, form = case
    if lens == "random":
        lens = torch.randint(1, L + 1, (B,), generator=torch.Generator().manual_seed(960 + seed)).tolist()
        lens[0] = L
    note("block scales seed=%d %s B=%d Hq=%d Hkv=%d nq=%d L=%d d=%d kv=%s S=%d lens=%s alibi=%s kb=%d vb=%d %s" %
         (seed, form, B, Hq, Hkv, nq, L, d, kv, S, lens, alibi, kb, vb, layout))
    c = block_case(940 + seed, B, Hq, Hkv, nq, L, d, kv, lens, alibi, kb, vb)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"], k_scale_block=kb, v_scale_block=vb)
    S = lib.resolve_splits(c["q"].to(DEV), c["k"].to(DEV), S)
    out = run_layout(lib, c, layout, S, kb, vb, "ws")
    two = run_layout(lib, c, layout, S, kb, vb, "split")
    alloc = run_layout(lib, c, layout, S, kb, vb, "alloc")
    torch.cuda.synchronize()
    assert torch.equal(out, two)
    assert torch.equal(out, alloc)
    vmax = vmax_valid(torch.from_numpy(dequantised(c["v"], c["v_scale"], vb)), c["seq_lens"])
    assert_parity(out.cpu().numpy(), ref, kv, vmax, "block scales %s" % form)


def test_block_scaled_partials_use_whole_blocks(lib):
    """With block scales the chunk length ceil(L / S) is rounded up to whole blocks
    (here 1000 keys, S = 7: 143 -> 256 with K blocks of 256, so chunks 4..6 are empty),
    and tad_split's partials are the chunk statistics of the dequantised values."""
    B, H, L, d, S, kb, vb = 1, 2, 1000, 128, 7, 256, 64
    c = block_case(990, B, H, H, 1, L, d, E4, None, False, kb, vb)
    g = {k: (x.to(DEV) if torch.is_tensor(x) else x) for k, x in c.items()}
    m, l, o = lib.split_partials(g["q"], g["k"], g["v"], None, None, S, k_scale=g["k_scale"],
                                 v_scale=g["v_scale"], k_scale_block=kb, v_scale_block=vb)
    torch.cuda.synchronize()
    m, l, o = m.cpu().double().numpy(), l.cpu().double().numpy(), o.cpu().double().numpy()
    kd, vd = dequantised(c["k"], c["k_scale"], kb), dequantised(c["v"], c["v_scale"], vb)
    clen = 256
    for h in range(H):
        parts = tree.chunk_partials(oracle.widen(c["q"])[0, h], kd[0, h], vd[0, h], S, None, clen)
        for s, (lm, den, num) in enumerate(parts):
            if den == 0.0:
                assert s >= 4 and m[0, h, s] == -np.inf and l[0, h, s] == 0
                continue
            assert m[0, h, s] * math.log(2) == pytest.approx(lm, rel=1e-5, abs=1e-5)
            fix = math.exp(m[0, h, s] * math.log(2) - lm)
            assert l[0, h, s] * fix == pytest.approx(den, rel=1e-4)
            np.testing.assert_allclose(o[0, h, s] * fix, num, rtol=2e-4, atol=2e-4 * np.abs(num).max())


def test_block_scaled_noalloc_shrinking(lib):
    """The allocation-free entry point with block scales: two calls in a row, the second
    smaller, each equal to tad_decode_ws bit for bit."""
    for seed, B, L, S in ((995, 2, 5000, 8), (996, 1, 1800, 4)):
        c = {k: (x.to(DEV) if torch.is_tensor(x) else x)
             for k, x in block_case(seed, B, 32, 8, 1, L, 128, E4, [L, L // 3][:B], False, 32, 64).items()}
        kw = dict(k_scale=c["k_scale"], v_scale=c["v_scale"], k_scale_block=32, v_scale_block=64)
        a = torch.empty((B, 32, 128), dtype=torch.float32, device=DEV)
        lib.tad_decode_noalloc(c["q"], c["k"], c["v"], c["seq_lens"], None, S, a, **kw)
        ws = lib.workspace(c["q"], c["k"], S)
        b = torch.empty_like(a)
        lib.tad_decode_ws(c["q"], c["k"], c["v"], c["seq_lens"], None, S, b, ws, **kw)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def draw_block_cases(n, seed=2026):
    """Random FP8 shapes with block scales on K, V or both (the other tensor then has one
    scale per (row, KV head)), on contiguous, token-major and paged caches."""
    rnd = random.Random(seed)
    cases = []
    for i in range(n):
        layout = rnd.choice(["contig", "tokmajor", "paged"])
        d = rnd.choice([64, 128, 128, 256] + ([512] if layout != "paged" else []))
        kv = rnd.choice([E4, E5])
        Hkv = rnd.choice([1, 2, 4, 8])
        group = rnd.choice([1, 1, 2, 4, 8])
        B = rnd.choice([1, 2, 3, 5, 8, 70])
        nq = rnd.choice([1, 1, 1, 2, 4])
        L = rnd.choice([1, 17, 300, 1000, 2500, 5000])
        if B * Hkv * group * L * d > 40_000_000:
            L = max(1, 40_000_000 // (B * Hkv * group * d))
        ragged = B > 1 and rnd.random() < 0.7
        S = rnd.choice([0, 0, 1, 3, 7, 8, 16, 24, 64])
        alibi = rnd.random() < 0.3
        blocks = [16, 32, 64, 128, 256, 1024]
        kb, vb = rnd.choice([0] + blocks), rnd.choice([0] + blocks)
        if kb == 0 and vb == 0:
            vb = rnd.choice(blocks)
        ps = rnd.choice([16, 32, 48, 64])
        cases.append((i, layout, B, Hkv * group, Hkv, nq, L, d, kv, ragged, S, alibi, kb, vb, ps))
    return cases


@pytest.mark.parametrize("case", draw_block_cases(40), ids=lambda c: "r%d-%s" % (c[0], c[1]))
def test_random_block_scaled(lib, case):
    i, layout, B, Hq, Hkv, nq, L, d, kv, ragged, S, alibi, kb, vb, ps = case
    lens = None
    if ragged:
        lens = torch.randint(0, L + 1, (B,), generator=torch.Generator().manual_seed(2700 + i)).tolist()
        lens[0], lens[-1] = L, 0
    elif layout == "paged":
        lens = [L] * B
    note("random block case %d: %s B=%d Hq=%d Hkv=%d nq=%d L=%d d=%d kv=%s lens=%s S=%d alibi=%s kb=%d vb=%d ps=%d"
         % (i, layout, B, Hq, Hkv, nq, L, d, kv, lens, S, alibi, kb, vb, ps))
    c = W.random_case(2800 + i, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi, scale_block=kb)
    if vb != kb:                                   # V in its own mode
        if vb:
            v, vs = W.draw_kv_fp8_blocks(2850 + i, B, Hkv, L, d, vb, kv)
        else:
            v, vs = W.draw_kv_fp8(2850 + i, B, Hkv, L, d, kv)
        if lens is not None:
            for b, Lb in enumerate(lens):
                v.view(torch.uint8)[b, :, Lb:, :] = 0x7F if kv == E4 else 0x7E
        c["v"], c["v_scale"] = v, vs
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(2900 + i))
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"], k_scale_block=kb, v_scale_block=vb)
    dv = lambda x: None if x is None else x.to(DEV)
    q, sl, sp = dv(c["q"]), dv(c["seq_lens"]), dv(c["slopes"])
    kw = dict(k_scale_block=kb, v_scale_block=vb)
    if layout == "paged":
        kc, vc, table = W.page_kv(c["k"], c["v"], ps, 2800 + i)
        Lcap = table.shape[1] * ps
        ks = dv(padded(c["k_scale"], kb, Lcap) if kb else c["k_scale"])
        vs = dv(padded(c["v_scale"], vb, Lcap) if vb else c["v_scale"])
        kc, vc, table = dv(kc), dv(vc), dv(table)
        out = lib.decode_paged(q, kc, vc, table, sl, sp, S, k_scale=ks, v_scale=vs, **kw)
        SS = S if S > 0 else lib.tad_auto_splits(B, Hq, Hkv, nq, Lcap, d, kc.dtype, 0)
        ws = lib.workspace(q, c["k"], SS)
        lib.tad_split_paged(q, kc, vc, table, sl, sp, SS, ws, k_scale=ks, v_scale=vs, **kw)
    else:
        if layout == "tokmajor":
            k = c["k"].view(torch.uint8).transpose(1, 2).contiguous().transpose(1, 2).view(kv).to(DEV)
            v = c["v"].view(torch.uint8).transpose(1, 2).contiguous().transpose(1, 2).view(kv).to(DEV)
        else:
            k, v = dv(c["k"]), dv(c["v"])
        ks, vs = dv(c["k_scale"]), dv(c["v_scale"])
        out = lib.decode(q, k, v, sl, sp, S, k_scale=ks, v_scale=vs, **kw)
        SS = lib.resolve_splits(q, k, S)
        ws = lib.workspace(q, k, SS)
        lib.tad_split(q, k, v, sl, sp, SS, ws, k_scale=ks, v_scale=vs, **kw)
    two = torch.full_like(out, float("nan"))
    lib.tad_combine(ws, B, Hq, nq, SS, d, two)
    torch.cuda.synchronize()
    assert torch.equal(out, two), "random block case %d: decode differs from split + combine" % i
    vd = dequantised(c["v"], c["v_scale"], vb) if vb else \
        np.nan_to_num(oracle.widen(c["v"])) * c["v_scale"].double().numpy()[:, :, None, None]
    assert_parity(out.cpu().numpy(), ref, kv, vmax_valid(torch.from_numpy(vd), c["seq_lens"]),
                  "random block case %d" % i)


@pytest.mark.parametrize("form", ["vector", "head-packed", "matrix cores"])
def test_block_scales_extreme_values(lib, form):
    """Block scales spanning 2^-30 .. 2^30, some exactly 0 (an all-zero block) and some
    negative (sign-flipped codes): scores reach ~1e10 and value rows ~1e11, and the
    result still matches the oracle (max-abs bar relative to the largest real |V|, and
    the rel-L2 gate)."""
    B, L, d, kb, vb = 2, 3000, 128, 32, 64
    Hq, Hkv = {"vector": (4, 4), "head-packed": (8, 8), "matrix cores": (16, 4)}[form]
    c = block_case(1100 + len(form), B, Hq, Hkv, 1, L, d, E4, [L, 1777], False, kb, vb)
    g = torch.Generator().manual_seed(1200 + len(form))
    for key in ("k_scale", "v_scale"):
        s = c[key]
        mag = torch.exp2(torch.randint(-30, 31, s.shape, generator=g).float())
        sign = torch.where(torch.rand(s.shape, generator=g) < 0.15, -1.0, 1.0)
        zero = torch.rand(s.shape, generator=g) < 0.05
        c[key] = torch.where(zero, torch.zeros_like(s), s * mag * sign).contiguous()
    note("extreme block scales %s: |scale| in [%g, %g]" % (form, c["v_scale"].abs()[c["v_scale"] != 0].min(),
                                                           c["v_scale"].abs().max()))
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], k_scale=c["k_scale"],
                            v_scale=c["v_scale"], k_scale_block=kb, v_scale_block=vb)
    layout = "tokmajor" if form == "head-packed" else "contig"
    out = run_layout(lib, c, layout, 6, kb, vb, "ws")
    two = run_layout(lib, c, layout, 6, kb, vb, "split")
    torch.cuda.synchronize()
    assert torch.equal(out, two)
    vmax = vmax_valid(torch.from_numpy(np.abs(dequantised(c["v"], c["v_scale"], vb))), c["seq_lens"])
    assert_parity(out.cpu().numpy(), ref, E4, vmax, "extreme block scales %s" % form)
