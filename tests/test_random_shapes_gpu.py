"""GPU parity on seeded random shapes: batch sizes across 64-row blocks, query-head
groups from 1 to 16, every head dimension and K/V dtype, ragged lengths with zeros,
1-3 query tokens, ALiBi, automatic and explicit chunk counts from 1 to 300, on
contiguous, token-major strided and paged caches.  Each case goes through the
workspace entry points (whichever kernel and merge form the library picks), is
compared with the fp64 oracle under the same bars as the other parity tests, and must
equal tad_split + tad_combine on the same inputs bit for bit (one launch or two, the
merge keeps the combine's arithmetic).
"""
import random

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_parity_gpu import DEV, assert_parity, note, vmax_real

pytestmark = pytest.mark.gpu

KV = [torch.float32, torch.bfloat16, torch.float8_e4m3fn, torch.float8_e5m2]


def draw_cases(n, seed=2024):
    rnd = random.Random(seed)
    cases = []
    for i in range(n):
        d = rnd.choice([64, 128, 128, 256, 512])
        kv = rnd.choice(KV)
        Hkv = rnd.choice([1, 2, 3, 4, 8])
        group = rnd.choice([1, 1, 2, 4, 8, 16])
        B = rnd.choice([1, 2, 3, 5, 8, 17, 70])
        nq = rnd.choice([1, 1, 1, 2, 3])
        L = rnd.choice([1, 7, 63, 300, 1000, 2500, 5000])
        if B * Hkv * group * L * d > 40_000_000:           # keep the oracle to a second or so
            L = max(1, 40_000_000 // (B * Hkv * group * d))
        ragged = B > 1 and rnd.random() < 0.7
        S = rnd.choice([0, 0, 1, 2, 3, 7, 16, 24, 64, 300])
        alibi = rnd.random() < 0.3
        cases.append((i, B, Hkv * group, Hkv, L, d, kv, nq, ragged, S, alibi))
    return cases


@pytest.mark.parametrize("case", draw_cases(80), ids=lambda c: "c%d" % c[0])
def test_random_shape(lib, case):
    i, B, Hq, Hkv, L, d, kv, nq, ragged, S, alibi = case
    g = torch.Generator().manual_seed(700 + i)
    lens = None
    if ragged:
        lens = torch.randint(0, L + 1, (B,), generator=g).tolist()
        lens[0] = L
        lens[-1] = 0
    note("random case %d: B=%d Hq=%d Hkv=%d L=%d d=%d kv=%s nq=%d lens=%s S=%d alibi=%s" %
         (i, B, Hq, Hkv, L, d, kv, nq, "ragged" if ragged else "none", S, alibi))
    c = W.random_case(800 + i, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi)
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(900 + i))
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"])
    gd = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in c.items()}
    out = lib.decode(gd["q"], gd["k"], gd["v"], gd["seq_lens"], gd["slopes"], S,
                     k_scale=gd["k_scale"], v_scale=gd["v_scale"])
    SS = lib.resolve_splits(gd["q"], gd["k"], S)
    ws = lib.workspace(gd["q"], gd["k"], SS)
    lib.tad_split(gd["q"], gd["k"], gd["v"], gd["seq_lens"], gd["slopes"], SS, ws, k_scale=gd["k_scale"],
                  v_scale=gd["v_scale"])
    sc = torch.full_like(out, float("nan"))
    lib.tad_combine(ws, B, Hq, nq, SS, d, sc)
    torch.cuda.synchronize()
    assert torch.equal(out, sc), "random case %d: decode differs from split + combine" % i
    assert_parity(out.cpu().numpy(), ref, kv, vmax_real(c), "random case %d" % i)


def draw_layout_cases(n, seed=2025):
    """Random shapes on token-major strided caches ([B, L, Hkv, d] storage seen as
    [B, Hkv, L, d]) and on paged caches (page sizes 16-128, pages stored token-major or
    head-major)."""
    rnd = random.Random(seed)
    cases = []
    for i in range(n):
        layout = rnd.choice(["tokmajor", "paged"])
        d = rnd.choice([64, 128, 128, 256] + ([512] if layout == "tokmajor" else []))
        kv = rnd.choice(KV if layout == "tokmajor" else KV[1:])
        Hkv = rnd.choice([1, 2, 3, 4, 8])
        group = rnd.choice([1, 1, 2, 4, 8, 16])
        B = rnd.choice([1, 2, 3, 5, 8, 17, 70])
        nq = rnd.choice([1, 1, 1, 2, 3])
        L = rnd.choice([1, 7, 16, 63, 300, 1000, 2500, 5000])
        if B * Hkv * group * L * d > 40_000_000:
            L = max(1, 40_000_000 // (B * Hkv * group * d))
        ragged = B > 1 and rnd.random() < 0.7
        S = rnd.choice([0, 0, 1, 2, 3, 7, 8, 9, 16, 24, 64, 300])
        alibi = rnd.random() < 0.3
        ps = rnd.choice([16, 32, 64, 128])
        head_major = rnd.random() < 0.5
        cases.append((i, layout, B, Hkv * group, Hkv, L, d, kv, nq, ragged, S, alibi, ps, head_major))
    return cases


def token_major(t):
    """The same values stored [B, L, Hkv, d], viewed as [B, Hkv, L, d] (byte-wise for FP8)."""
    if t.element_size() == 1:
        return t.view(torch.uint8).transpose(1, 2).contiguous().transpose(1, 2).view(t.dtype)
    return t.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("case", draw_layout_cases(60), ids=lambda c: "l%d-%s" % (c[0], c[1]))
def test_random_layout(lib, case):
    i, layout, B, Hq, Hkv, L, d, kv, nq, ragged, S, alibi, ps, head_major = case
    g = torch.Generator().manual_seed(1700 + i)
    lens = None
    if ragged:
        lens = torch.randint(0, L + 1, (B,), generator=g).tolist()
        lens[0] = L
        lens[-1] = 0
    elif layout == "paged":
        lens = [L] * B                 # without seq_lens a paged row spans all its pages
    note("random layout case %d: %s B=%d Hq=%d Hkv=%d L=%d d=%d kv=%s nq=%d ragged=%s S=%d alibi=%s ps=%d hm=%s" %
         (i, layout, B, Hq, Hkv, L, d, kv, nq, ragged, S, alibi, ps, head_major))
    c = W.random_case(1800 + i, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi)
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(1900 + i))
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"])
    dv = lambda x: None if x is None else x.to(DEV)
    q, sl, sp, ks, vs = dv(c["q"]), dv(c["seq_lens"]), dv(c["slopes"]), dv(c["k_scale"]), dv(c["v_scale"])
    if layout == "paged":
        kc, vc, table = W.page_kv(c["k"], c["v"], ps, 1800 + i, head_major=head_major)
        kc, vc, table = dv(kc), dv(vc), dv(table)
        out = lib.decode_paged(q, kc, vc, table, sl, sp, S, k_scale=ks, v_scale=vs)
        # the paged entry point's automatic count sees whole pages: table width x page size
        SS = S if S > 0 else lib.tad_auto_splits(B, Hq, Hkv, nq, table.shape[1] * kc.shape[1], d, kc.dtype, 0)
        ws = lib.workspace(q, c["k"], SS)
        lib.tad_split_paged(q, kc, vc, table, sl, sp, SS, ws, k_scale=ks, v_scale=vs)
    else:
        k, v = dv(token_major(c["k"])), dv(token_major(c["v"]))
        out = lib.decode(q, k, v, sl, sp, S, k_scale=ks, v_scale=vs)
        SS = lib.resolve_splits(q, k, S)
        ws = lib.workspace(q, k, SS)
        lib.tad_split(q, k, v, sl, sp, SS, ws, k_scale=ks, v_scale=vs)
    sc = torch.full_like(out, float("nan"))
    lib.tad_combine(ws, B, Hq, nq, SS, d, sc)
    torch.cuda.synchronize()
    assert torch.equal(out, sc), "random layout case %d: decode differs from split + combine" % i
    assert_parity(out.cpu().numpy(), ref, kv, vmax_real(c), "random layout case %d" % i)
