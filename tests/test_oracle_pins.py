"""Pins for the fp64 oracle: truths that do not come from the oracle itself.

Each test fixes the oracle against a closed form, an invariant of softmax attention,
a value printed on the pages, a library attention routine, or the split-and-merge
steps of the tree-attention gist (a different algorithm reaching the same result).
A plausible slip in the oracle -- a dropped scale, a wrong bias sign, a transposed
operand, a wrong head mapping, a missed max-subtraction, a length off by one --
fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import tree
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(x):
    return oracle.widen(x)


def rand_case(seed, B=1, Hq=1, Hkv=1, L=31, d=16, kv=torch.float32, **kw):
    return W.random_case(seed, B, Hq, Hkv, L, d, q_dtype=torch.float32, kv_dtype=kv, **kw)


# ----------------------------------------------------------------------------- printed values

def test_alibi_bias_matches_printed_row():
    """The causal ALiBi row printed for seq_len 5 is [-4, -3, -2, -1, 0]."""
    with open(os.path.join(GOLDEN, "alibi_causal_row_L5.txt")) as f:
        lines = [ln for ln in f if not ln.startswith("#") and ln.strip()]
    L = int(lines[0])
    expect = [float(x) for x in lines[1].split()]
    got = [oracle.alibi_bias(L, j, 1.0) for j in range(L)]
    assert got == expect
    # the head constant multiplies the whole row
    assert [oracle.alibi_bias(L, j, 0.25) for j in range(L)] == [0.25 * e for e in expect]


# ----------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("kv", [torch.float32, torch.bfloat16])
def test_zero_query_gives_mean_of_values(kv):
    c = rand_case(1, B=2, Hq=3, Hkv=3, L=37, d=32, kv=kv)
    c["q"].zero_()
    out = oracle.decode_f64(c["q"], c["k"], c["v"])
    np.testing.assert_allclose(out, f64(c["v"]).mean(axis=2), rtol=0, atol=1e-14)


def test_zero_query_alibi_geometric_closed_form():
    """q = 0 with ALiBi: weights r^(L-1-j), r = e^(-slope).  With v_j = j (every dim)
    the output is ((L-1) S0 - S1) / S0, S0 = sum r^i = (1-r^L)/(1-r),
    S1 = sum i r^i = r (1 - L r^(L-1) + (L-1) r^L) / (1-r)^2."""
    B, H, L, d = 1, 4, 53, 8
    q = torch.zeros(B, H, d)
    k = torch.randn(B, H, L, d, generator=torch.Generator().manual_seed(5))
    v = torch.arange(L, dtype=torch.float32).view(1, 1, L, 1).expand(B, H, L, d).contiguous()
    slopes = W.alibi_slopes(H)
    out = oracle.decode_f64(q, k, v, slopes=slopes)
    for h in range(H):
        a = float(slopes[h])
        r = math.exp(-a)
        one_minus_r = -math.expm1(-a)          # 1 - r without cancellation
        S0 = -math.expm1(-a * L) / one_minus_r
        S1 = r * (1 - L * r ** (L - 1) + (L - 1) * r ** L) / one_minus_r ** 2
        expect = ((L - 1) * S0 - S1) / S0
        # the closed form's own rounding (S1's bracket cancels for small slopes) is ~1e-12
        np.testing.assert_allclose(out[0, h], expect, rtol=1e-11)
        # later keys weigh more: the mean position exceeds the unbiased mean (L-1)/2
        assert expect > (L - 1) / 2


def test_two_keys_sigmoid():
    """Two keys: out = sigmoid(s1 - s2) v1 + sigmoid(s2 - s1) v2, s_i = q.k_i / sqrt(d)."""
    d = 16
    q = torch.zeros(1, 1, d)
    q[0, 0, 0] = 2.0
    q[0, 0, 3] = -1.0
    k = torch.zeros(1, 1, 2, d)
    k[0, 0, 0, 0] = 1.5      # q.k1 = 3
    k[0, 0, 1, 3] = 0.5      # q.k2 = -0.5
    v = torch.randn(1, 1, 2, d, generator=torch.Generator().manual_seed(2))
    s1, s2 = 3.0 / math.sqrt(d), -0.5 / math.sqrt(d)
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    expect = sig(s1 - s2) * f64(v)[0, 0, 0] + sig(s2 - s1) * f64(v)[0, 0, 1]
    out = oracle.decode_f64(q, k, v)
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-14, atol=1e-15)


def test_single_key_returns_its_value():
    c = rand_case(3, L=1, d=8)
    out = oracle.decode_f64(c["q"], c["k"], c["v"])
    np.testing.assert_array_equal(out[0, 0], f64(c["v"])[0, 0, 0])


@pytest.mark.parametrize("score", [60.0, 100.0, 800.0])
def test_dominant_key_returns_its_value(score):
    """One key scoring `score` above a bulk of small scores: output is that key's value.
    score=800 would overflow exp() without the max subtraction."""
    B, H, L, d = 1, 2, 257, 64
    g = torch.Generator().manual_seed(9)
    q = torch.randn(B, H, d, generator=g)
    k = 0.01 * torch.randn(B, H, L, d, generator=g)
    v = torch.randn(B, H, L, d, generator=g)
    p = [17, 250]
    for h in range(H):
        qh = q[0, h].double()
        k[0, h, p[h]] = (score * math.sqrt(d) / float(qh @ qh) * qh).float()
    out = oracle.decode_f64(q, k, v)
    for h in range(H):
        assert np.isfinite(out[0, h]).all()
        np.testing.assert_allclose(out[0, h], f64(v)[0, h, p[h]], rtol=0, atol=1e-20 + 1e-15 * (score < 100))


def test_empty_sequence_gives_zero():
    c = rand_case(4, B=2, L=9, d=8, seq_lens=[0, 9])
    out = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"])
    assert (out[0] == 0).all()
    assert np.isfinite(out[1]).all() and (out[1] != 0).any()


# ----------------------------------------------------------------------------- invariants

def test_constant_value_rows():
    c = rand_case(5, L=40, d=16)
    row = torch.randn(16, generator=torch.Generator().manual_seed(50))
    v = row.view(1, 1, 1, 16).expand(1, 1, 40, 16).contiguous()
    out = oracle.decode_f64(c["q"], c["k"], v)
    np.testing.assert_allclose(out[0, 0], f64(row), rtol=1e-14, atol=1e-15)


def test_value_shift_and_linearity():
    c = rand_case(6, B=1, Hq=2, Hkv=2, L=45, d=16)
    c["v"] = torch.round(c["v"] * 64) / 64      # on a 1/64 grid: v + 3 is exact in fp32
    base = oracle.decode_f64(c["q"], c["k"], c["v"])
    shifted = oracle.decode_f64(c["q"], c["k"], c["v"] + 3.0)
    np.testing.assert_allclose(shifted, base + 3.0, rtol=0, atol=1e-13)
    v2 = torch.randn(c["v"].shape, generator=torch.Generator().manual_seed(60))
    o2 = oracle.decode_f64(c["q"], c["k"], v2)
    comb = oracle.decode_f64(c["q"], c["k"], (2.0 * c["v"].double() - 0.5 * v2.double()).float())
    np.testing.assert_allclose(comb, 2.0 * base - 0.5 * o2, rtol=0, atol=1e-6)  # fp32 input rounding


def test_key_permutation_invariance():
    c = rand_case(7, B=1, Hq=2, Hkv=2, L=50, d=16)
    perm = torch.randperm(50, generator=torch.Generator().manual_seed(70))
    out = oracle.decode_f64(c["q"], c["k"], c["v"])
    outp = oracle.decode_f64(c["q"], c["k"][:, :, perm].contiguous(), c["v"][:, :, perm].contiguous())
    np.testing.assert_allclose(outp, out, rtol=1e-13, atol=1e-15)


def test_score_shift_invariance():
    """Adding the same vector u to every key adds q.u/sqrt(d) to every score: no change
    (softmax is shift invariant, the point of the ALiBi thread's answer)."""
    c = rand_case(8, B=1, Hq=3, Hkv=3, L=33, d=16, kv=torch.float32)
    c["k"] = torch.round(c["k"] * 64) / 64      # on a 1/64 grid: k + u is exact in fp32
    u = torch.zeros(16)
    u[[1, 5]] = 0.5    # exactly representable shift of every key
    out = oracle.decode_f64(c["q"], c["k"], c["v"])
    out2 = oracle.decode_f64(c["q"], c["k"] + u, c["v"])
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)


def test_scale_is_inverse_sqrt_head_dim():
    """Scaling q by sqrt(d) removes the d^-1/2 scale: compare with softmax(q.k) V directly
    on a two-key case computed by hand (different d give different outputs)."""
    for d in (4, 64):
        q = torch.zeros(1, 1, d)
        q[0, 0, 0] = 1.0
        k = torch.zeros(1, 1, 2, d)
        k[0, 0, 0, 0] = 2.0
        v = torch.zeros(1, 1, 2, d)
        v[0, 0, 0, 0] = 1.0
        out = oracle.decode_f64(q, k, v)
        w0 = math.exp(2.0 / math.sqrt(d)) / (math.exp(2.0 / math.sqrt(d)) + 1.0)
        assert abs(out[0, 0, 0] - w0) < 1e-15


# ----------------------------------------------------------------------------- library routine

@pytest.mark.parametrize("alibi", [False, True])
@pytest.mark.parametrize("kv", [torch.float32, torch.bfloat16])
def test_matches_torch_sdpa_fp64(alibi, kv):
    """torch's scaled_dot_product_attention in fp64, GQA expanded by repeat_interleave,
    ALiBi and lengths passed as a float mask."""
    B, Hq, Hkv, L, d = 3, 8, 2, 70, 32
    lens = [70, 1, 33]
    c = rand_case(10, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, kv=kv, seq_lens=lens, alibi=alibi)
    out = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"])
    q = torch.from_numpy(f64(c["q"])).unsqueeze(2)                      # [B,Hq,1,d]
    k = torch.from_numpy(np.nan_to_num(f64(c["k"]))).repeat_interleave(Hq // Hkv, dim=1)
    v = torch.from_numpy(np.nan_to_num(f64(c["v"]))).repeat_interleave(Hq // Hkv, dim=1)
    mask = torch.full((B, Hq, 1, L), -math.inf, dtype=torch.float64)
    for b, Lb in enumerate(lens):
        j = torch.arange(Lb, dtype=torch.float64)
        bias = torch.zeros(Hq, Lb, dtype=torch.float64)
        if alibi:
            bias = -c["slopes"].double().view(Hq, 1) * (Lb - 1 - j).view(1, Lb)
        mask[b, :, 0, :Lb] = bias
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask).squeeze(2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- structure

def test_gqa_equals_mha_with_repeated_kv():
    c = rand_case(11, B=2, Hq=8, Hkv=2, L=29, d=16)
    out = oracle.decode_f64(c["q"], c["k"], c["v"])
    k4 = c["k"].repeat_interleave(4, dim=1).contiguous()
    v4 = c["v"].repeat_interleave(4, dim=1).contiguous()
    ref = oracle.decode_f64(c["q"], k4, v4)
    np.testing.assert_array_equal(out, ref)
    # a modulo head mapping would differ
    kmod = c["k"].repeat(1, 4, 1, 1).contiguous()
    vmod = c["v"].repeat(1, 4, 1, 1).contiguous()
    assert not np.allclose(oracle.decode_f64(c["q"], kmod, vmod), out)


@pytest.mark.parametrize("alibi", [False, True])
def test_ragged_equals_truncated(alibi):
    lens = [5, 40, 23]
    c = rand_case(12, B=3, Hq=4, Hkv=4, L=40, d=16, seq_lens=lens, alibi=alibi)
    out = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"])
    assert np.isfinite(out).all()          # NaN tail never read
    for b, Lb in enumerate(lens):
        ref = oracle.decode_f64(c["q"][b:b + 1], c["k"][b:b + 1, :, :Lb], c["v"][b:b + 1, :, :Lb],
                                slopes=c["slopes"])
        np.testing.assert_array_equal(out[b], ref[0])


def test_rows_subset_and_strides():
    c = rand_case(13, B=2, Hq=4, Hkv=2, L=30, d=16)
    full = oracle.decode_f64(c["q"], c["k"], c["v"])
    rows = [7, 0, 5]
    sub = oracle.decode_f64(c["q"], c["k"], c["v"], rows=rows)
    for i, r in enumerate(rows):
        np.testing.assert_array_equal(sub[i], full[r // 4, r % 4])
    # a [B, L, H, d] cache viewed as [B, H, L, d] (non-contiguous key stride)
    kt = c["k"].transpose(1, 2).contiguous().transpose(1, 2)
    vt = c["v"].transpose(1, 2).contiguous().transpose(1, 2)
    np.testing.assert_array_equal(oracle.decode_f64(c["q"], kt, vt), full)


def test_bf16_widening_matches_torch():
    x = torch.randn(1000, generator=torch.Generator().manual_seed(14)).to(torch.bfloat16)
    x[0] = float("inf")
    x[1] = -0.0
    np.testing.assert_array_equal(oracle.widen(x), x.to(torch.float64).numpy())


# ----------------------------------------------------------------------------- split + merge

@pytest.mark.parametrize("n_chunks", [1, 2, 3, 7, 8, 31, 36])
@pytest.mark.parametrize("alibi", [False, True])
def test_tree_decode_matches_definition(n_chunks, alibi):
    """The gist's own test shape: 31 keys of width 512 over 8 ranks (chunks 4,...,4,3),
    plus other chunk counts, including more chunks than keys (empty chunks)."""
    L, d = 31, 512
    c = rand_case(15, B=1, Hq=2, Hkv=2, L=L, d=d, alibi=alibi)
    out = oracle.decode_f64(c["q"], c["k"], c["v"], slopes=c["slopes"])
    for h in range(2):
        bias = None
        if alibi:
            bias = np.array([oracle.alibi_bias(L, j, float(c["slopes"][h])) for j in range(L)])
        got = tree.tree_decode_row(f64(c["q"])[0, h], f64(c["k"])[0, h], f64(c["v"])[0, h],
                                   n_chunks, bias)
        np.testing.assert_allclose(got, out[0, h], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("chunk_len", [1, 5, 13, 40, 100])
def test_fixed_chunk_length_matches_definition(chunk_len):
    """A batch-wide chunk length (rows ending in empty chunks) gives the same result."""
    L, d = 77, 32
    c = rand_case(18, L=L, d=d, alibi=True)
    out = oracle.decode_f64(c["q"], c["k"], c["v"], slopes=c["slopes"])
    bias = np.array([oracle.alibi_bias(L, j, float(c["slopes"][0])) for j in range(L)])
    n = max(1, -(-100 // chunk_len))
    got = tree.tree_decode_row(f64(c["q"])[0, 0], f64(c["k"])[0, 0], f64(c["v"])[0, 0], n, bias, chunk_len)
    np.testing.assert_allclose(got, out[0, 0], rtol=1e-12, atol=1e-14)
    assert tree.chunk_bounds(L, 3, 40) == [(0, 40), (40, 77), (77, 77)]


def test_gist_chunk_sizes():
    """torch.chunk semantics: 31 keys over 8 -> seven chunks of 4 and one of 3;
    9 keys over 8 -> chunk length 2, five non-empty chunks and three empty ones."""
    assert [hi - lo for lo, hi in tree.chunk_bounds(31, 8)] == [4] * 7 + [3]
    assert [hi - lo for lo, hi in tree.chunk_bounds(9, 8)] == [2, 2, 2, 2, 1, 0, 0, 0]
    sizes = [t.shape[0] for t in torch.arange(31).chunk(8)]
    assert sizes == [4] * 7 + [3]


def test_merge_order_and_tree_shape_invariance():
    L, d = 300, 64
    c = rand_case(16, L=L, d=d, k_scale=3.0)
    q, k, v = f64(c["q"])[0, 0], f64(c["k"])[0, 0], f64(c["v"])[0, 0]
    ref = oracle.decode_f64(c["q"], c["k"], c["v"])[0, 0]
    parts = tree.chunk_partials(q, k, v, 13)
    rng = np.random.default_rng(0)
    for _ in range(5):
        order = rng.permutation(13)
        np.testing.assert_allclose(tree.merge_all(parts, order), ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(tree.merge_tree(parts, order), ref, rtol=1e-12, atol=1e-14)


def test_partials_are_local_softmax_statistics():
    """Each chunk summary (peak, mass, vsum) is pinned by two independent routes: vsum /
    mass is the plain decode over the chunk's keys alone (the C oracle on the sliced
    K and V), and peak + log(mass) is the log-sum-exp of the chunk's scores (scipy).
    The peak is the chunk's largest score.  These are the quantities the GPU split
    kernel stores (with the peak in base 2)."""
    from scipy.special import logsumexp
    L, d = 50, 16
    c = rand_case(17, L=L, d=d)
    q, k, v = f64(c["q"])[0, 0], f64(c["k"])[0, 0], f64(c["v"])[0, 0]
    parts = tree.chunk_partials(q, k, v, 4)
    s = k @ q / math.sqrt(d)
    for (lo, hi), (m, den, num) in zip(tree.chunk_bounds(L, 4), parts):
        assert m == pytest.approx(s[lo:hi].max(), rel=1e-15)
        assert m + math.log(den) == pytest.approx(float(logsumexp(s[lo:hi])), rel=1e-13)
        chunk_out = oracle.decode_f64(c["q"], c["k"][:, :, lo:hi].contiguous(), c["v"][:, :, lo:hi].contiguous())
        np.testing.assert_allclose(num / den, chunk_out[0, 0], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- workload recipes

def test_planted_key_dominates_stress_recipe():
    """The 1M-key workload's planted key (logit ~ +60 among bf16(6 N(0,1)) keys)
    dominates: on a 2^14-key slice built by the same recipe the output is that key's
    V row to ~1e-12."""
    B, H, L, d = 1, 2, 1 << 14, 128
    q = W.draw_q(77, B, H, d)
    k = W.draw_kv(78, B, H, L, d, torch.bfloat16, 6.0)
    v = W.draw_kv(79, B, H, L, d, torch.bfloat16)
    pos = W.plant_dominant_keys(80, q, k, 60.0)
    out = oracle.decode_f64(q, k, v)
    for h in range(H):
        np.testing.assert_allclose(out[0, h], f64(v)[0, h, int(pos[0, h])], rtol=0, atol=1e-9)


def test_workload_recipes_shapes():
    w = W.WORKLOADS[3]
    sl = W.draw_seq_lens(3003, w.B, w.ragged_lo, w.Lmax)
    assert sl.dtype == torch.int32 and sl.min() >= 1024 and sl.max() <= 32768
    s = W.alibi_slopes(16)
    assert s[0] == 2 ** -0.5 and s[15] == 2 ** -8
    assert W.WORKLOADS[2].kv_bytes() == 2 * 1024 ** 3


# ----------------------------------------------------------------------------- fp8

@pytest.mark.parametrize("fmt,tdt", [(oracle.FP8_E4M3, torch.float8_e4m3fn), (oracle.FP8_E5M2, torch.float8_e5m2)])
def test_fp8_decoding_matches_torch(fmt, tdt):
    """The oracle's OCP FP8 decoding equals torch's float8 types for all 256 patterns."""
    ref = torch.arange(256, dtype=torch.uint8).view(tdt).to(torch.float64).numpy()
    got = np.array([oracle.fp8_value(i, fmt) for i in range(256)])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_fp8_known_values():
    e4 = lambda b: oracle.fp8_value(b, oracle.FP8_E4M3)
    e5 = lambda b: oracle.fp8_value(b, oracle.FP8_E5M2)
    assert e4(0x7E) == 448.0 and e4(0x01) == 2.0 ** -9 and e4(0x38) == 1.0 and e4(0xB8) == -1.0
    assert math.isnan(e4(0x7F)) and math.isnan(e4(0xFF))
    assert e5(0x7B) == 57344.0 and e5(0x01) == 2.0 ** -16 and e5(0x3C) == 1.0
    assert e5(0x7C) == math.inf and math.isnan(e5(0x7E))


@pytest.mark.parametrize("tdt", [torch.float8_e4m3fn, torch.float8_e5m2])
def test_fp8_scaled_equals_dequantised_fp32(tdt):
    """FP8 K/V with per-(b, head) scales give the output of the dequantised values
    (stored * scale, exact in fp32 for these scales' products)."""
    c = W.random_case(19, B=2, Hq=4, Hkv=2, L=60, d=32, kv_dtype=tdt)
    out = oracle.decode_f64(c["q"], c["k"], c["v"], k_scale=c["k_scale"], v_scale=c["v_scale"])
    kd = torch.from_numpy(oracle.widen(c["k"]) * c["k_scale"].double().numpy()[:, :, None, None])
    vd = torch.from_numpy(oracle.widen(c["v"]) * c["v_scale"].double().numpy()[:, :, None, None])
    q = torch.from_numpy(f64(c["q"])).unsqueeze(2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, kd.repeat_interleave(2, dim=1), vd.repeat_interleave(2, dim=1)).squeeze(2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)
    # the scales matter: without them the output differs
    assert not np.allclose(oracle.decode_f64(c["q"], c["k"], c["v"]), out)


def block_dequantised(codes, scales, block):
    """fp64 real values of FP8 codes [B, H, L, d] under block scales [B, H, nblk]: each
    scale repeated over its block's key positions (numpy's repeat, then cut to L)."""
    L = codes.shape[2]
    rep = np.repeat(scales.double().numpy(), block, axis=2)[:, :, :L]
    return np.nan_to_num(oracle.widen(codes)) * rep[:, :, :, None]


@pytest.mark.parametrize("alibi", [False, True])
@pytest.mark.parametrize("tdt", [torch.float8_e4m3fn, torch.float8_e5m2])
def test_fp8_block_scales_match_sdpa_on_dequantised(tdt, alibi):
    """FP8 K/V with one scale per block of key positions (K blocks of 16, V blocks of 32;
    75 keys, so both last blocks are partial; ragged lengths, GQA) give torch's fp64
    scaled_dot_product_attention over the dequantised values."""
    B, Hq, Hkv, L, d, kb, vb = 3, 8, 2, 75, 32, 16, 32
    lens = [75, 17, 40]
    c = W.random_case(23, B, Hq, Hkv, L, d, kv_dtype=tdt, seq_lens=lens, alibi=alibi)
    k, ks = W.draw_kv_fp8_blocks(24, B, Hkv, L, d, kb, tdt)
    v, vs = W.draw_kv_fp8_blocks(25, B, Hkv, L, d, vb, tdt)
    out = oracle.decode_f64(c["q"], k, v, seq_lens=c["seq_lens"], slopes=c["slopes"], k_scale=ks, v_scale=vs,
                            k_scale_block=kb, v_scale_block=vb)
    q = torch.from_numpy(f64(c["q"])).unsqueeze(2)
    kd = torch.from_numpy(block_dequantised(k, ks, kb)).repeat_interleave(Hq // Hkv, dim=1)
    vd = torch.from_numpy(block_dequantised(v, vs, vb)).repeat_interleave(Hq // Hkv, dim=1)
    mask = torch.full((B, Hq, 1, L), -math.inf, dtype=torch.float64)
    for b, Lb in enumerate(lens):
        j = torch.arange(Lb, dtype=torch.float64)
        bias = torch.zeros(Hq, Lb, dtype=torch.float64)
        if alibi:
            bias = -c["slopes"].double().view(Hq, 1) * (Lb - 1 - j).view(1, Lb)
        mask[b, :, 0, :Lb] = bias
    ref = torch.nn.functional.scaled_dot_product_attention(q, kd, vd, attn_mask=mask).squeeze(2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)
    # the block index matters: one block off, or K and V blocks swapped, differ
    ks_shift = torch.roll(ks, 1, dims=2)
    assert not np.allclose(oracle.decode_f64(c["q"], k, v, seq_lens=c["seq_lens"], slopes=c["slopes"],
                                             k_scale=ks_shift, v_scale=vs, k_scale_block=kb,
                                             v_scale_block=vb), out)


def test_fp8_block_scales_zero_query_closed_form():
    """q = 0: every visible key weighs the same, so the output is the mean of the
    dequantised value rows of the row's first L_b keys (V blocks of 64 over 150 keys)."""
    B, Hkv, L, d, vb = 2, 2, 150, 16, 64
    lens = [150, 70]
    c = W.random_case(26, B, 2 * Hkv, Hkv, L, d, kv_dtype=torch.float8_e4m3fn, seq_lens=lens,
                      scale_block=vb)
    q = torch.zeros_like(c["q"])
    out = oracle.decode_f64(q, c["k"], c["v"], seq_lens=c["seq_lens"], k_scale=c["k_scale"],
                            v_scale=c["v_scale"], k_scale_block=vb, v_scale_block=vb)
    vd = block_dequantised(c["v"], c["v_scale"], vb)
    for b, Lb in enumerate(lens):
        for h in range(2 * Hkv):
            np.testing.assert_allclose(out[b, h], vd[b, h // 2, :Lb].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_fp8_block_scales_constant_equal_head_scales():
    """Block scales that repeat the (b, head) scale in every block give exactly the
    per-(b, head) result."""
    c = W.random_case(27, B=2, Hq=4, Hkv=2, L=50, d=16, kv_dtype=torch.float8_e4m3fn)
    out = oracle.decode_f64(c["q"], c["k"], c["v"], k_scale=c["k_scale"], v_scale=c["v_scale"])
    kb = c["k_scale"][:, :, None].repeat(1, 1, 4).contiguous()
    vb = c["v_scale"][:, :, None].repeat(1, 1, 2).contiguous()
    blk = oracle.decode_f64(c["q"], c["k"], c["v"], k_scale=kb, v_scale=vb, k_scale_block=16, v_scale_block=32)
    np.testing.assert_array_equal(out, blk)


# ----------------------------------------------------------------------------- several query tokens

def multi_case(seed, B, Hq, Hkv, nq, L, d, lens=None, alibi=False):
    c = W.random_case(seed, B, Hq, Hkv, L, d, seq_lens=lens, alibi=alibi)
    c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(seed + 9))
    return c


@pytest.mark.parametrize("alibi", [False, True])
def test_multi_token_matches_sdpa_with_causal_mask(alibi):
    """nq new tokens at the last nq positions, each seeing the keys up to its own
    position: torch SDPA (fp64) with an explicit causal mask (and the ALiBi term
    -slope * (position - j)) over those query positions."""
    B, Hq, Hkv, nq, L, d = 2, 4, 2, 5, 40, 16
    lens = [40, 23]
    c = multi_case(21, B, Hq, Hkv, nq, L, d, lens, alibi)
    out = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"])
    assert out.shape == (B, Hq, nq, d)
    q = torch.from_numpy(f64(c["q"]))
    k = torch.from_numpy(np.nan_to_num(f64(c["k"]))).repeat_interleave(Hq // Hkv, dim=1)
    v = torch.from_numpy(np.nan_to_num(f64(c["v"]))).repeat_interleave(Hq // Hkv, dim=1)
    mask = torch.full((B, Hq, nq, L), -math.inf, dtype=torch.float64)
    for b, Lb in enumerate(lens):
        for t in range(nq):
            pos = Lb - nq + t
            j = torch.arange(pos + 1, dtype=torch.float64)
            bias = torch.zeros(Hq, pos + 1, dtype=torch.float64)
            if alibi:
                bias = -c["slopes"].double().view(Hq, 1) * (pos - j).view(1, -1)
            mask[b, :, t, :pos + 1] = bias
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_multi_token_last_token_is_single_token_decode():
    """The last of nq tokens sees every key: it equals single-token decode with that q;
    a single token given in 4-D form equals the 3-D form."""
    c = multi_case(22, 2, 4, 4, 3, 50, 32, [50, 31])
    out = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"])
    single = oracle.decode_f64(c["q"][:, :, -1].contiguous(), c["k"], c["v"], seq_lens=c["seq_lens"])
    np.testing.assert_array_equal(out[:, :, -1], single)
    one = oracle.decode_f64(c["q"][:, :, :1].contiguous(), c["k"], c["v"], seq_lens=c["seq_lens"])
    np.testing.assert_array_equal(one[:, :, 0], oracle.decode_f64(c["q"][:, :, 0].contiguous(), c["k"], c["v"],
                                                                    seq_lens=c["seq_lens"]))


def test_multi_token_more_tokens_than_keys():
    """Tokens whose position is before the first key see nothing: output 0."""
    c = multi_case(23, 1, 2, 2, 6, 4, 16)
    out = oracle.decode_f64(c["q"], c["k"], c["v"])
    assert (out[:, :, :2] == 0).all()                    # positions -2, -1
    assert np.isfinite(out).all() and (out[:, :, 2:] != 0).any()


@pytest.mark.parametrize("g,alibi,ragged", [(1, False, False), (1, True, False), (2, False, True),
                                            (2, True, True)])
def test_brute_force_50_digits(g, alibi, ragged):
    """The definition evaluated independently in 50-digit arithmetic (mpmath) on tiny
    inputs -- scores d^-1/2 q.k plus the bias -slope (L - 1 - j), the exact softmax over
    the row's L keys, the weighted sum of value rows -- matches the oracle to 1e-13
    relative.  Covers MHA and two query heads per KV head, ALiBi, and ragged rows with
    an empty one."""
    mpmath = pytest.importorskip("mpmath")
    mp = mpmath.mp
    mp.dps = 50
    B, Hkv, L, d = 3, 2, 13, 8
    Hq = Hkv * g
    lens = [13, 5, 0] if ragged else None
    c = W.random_case(4200 + 10 * g + 2 * alibi + ragged, B, Hq, Hkv, L, d, kv_dtype=torch.float32,
                      seq_lens=lens, alibi=alibi)
    q, k, v = f64(c["q"]), f64(c["k"]), f64(c["v"])
    slopes = None if c["slopes"] is None else c["slopes"].double().numpy()
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"])
    scale = 1 / mpmath.sqrt(d)
    for b in range(B):
        Lb = L if lens is None else lens[b]
        for h in range(Hq):
            kvh = h // g
            if Lb == 0:
                assert (ref[b, h] == 0).all()
                continue
            s = []
            for j in range(Lb):
                x = scale * mpmath.fsum(mpmath.mpf(float(q[b, h, i])) * mpmath.mpf(float(k[b, kvh, j, i]))
                                        for i in range(d))
                if slopes is not None:
                    x -= mpmath.mpf(float(slopes[h])) * (Lb - 1 - j)
                s.append(x)
            top = max(s)
            w = [mpmath.exp(x - top) for x in s]
            z = mpmath.fsum(w)
            want = np.array([float(mpmath.fsum(w[j] * mpmath.mpf(float(v[b, kvh, j, e])) for j in range(Lb)) / z)
                             for e in range(d)])
            np.testing.assert_allclose(ref[b, h], want, rtol=1e-13, atol=1e-13 * np.abs(want).max())
