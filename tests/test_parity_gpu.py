"""GPU parity: libtad (through its C ABI) against the fp64 oracle.

Bars (the acceptance tolerances of the method): fp32 K/V -> max-abs error <= 1e-5;
bf16 K/V (fp32 accumulation) -> max-abs error <= 2e-3 * max|V| over the valid keys.
A stricter diagnostic also holds every case to a relative L2 error <= 1e-4, so that a
subtly wrong kernel cannot hide under the loose bf16 bar (long-context outputs are
averages of many rows and are small).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import tree
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_L2_DIAG = 1e-4


def note(msg):
    print("[case] " + msg, flush=True)


def vmax_valid(v, seq_lens):
    vv = v.float()
    if seq_lens is None:
        return float(vv.abs().max())
    return max(float(vv[b, :, :max(0, int(L))].abs().max()) if int(L) > 0 else 0.0
               for b, L in enumerate(seq_lens))


def assert_parity(out, ref, kv_dtype, vmax, what=""):
    out = np.asarray(out, dtype=np.float64)
    err = np.abs(out - ref)
    max_abs = float(err.max()) if err.size else 0.0
    bar = 1e-5 if kv_dtype == torch.float32 else 2e-3 * vmax
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(out - ref)) / nref if nref > 0 else float(np.linalg.norm(out))
    note("%s max_abs=%.3e bar=%.3e rel_l2=%.3e" % (what, max_abs, bar, rel))
    assert np.isfinite(out).all(), what
    assert max_abs <= bar, (what, max_abs, bar)
    assert rel <= REL_L2_DIAG, (what, rel)


def to_dev(c):
    g = dict(c)
    for key in ("q", "k", "v", "seq_lens", "slopes", "k_scale", "v_scale"):
        if g.get(key) is not None:
            g[key] = g[key].to(DEV)
    return g


def gpu_decode(lib, c, n_splits):
    g = to_dev(c)
    out = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], n_splits,
                     k_scale=g.get("k_scale"), v_scale=g.get("v_scale"))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def vmax_real(c):
    """max |V| over valid keys, in real (dequantised) units."""
    v = torch.from_numpy(oracle.widen(c["v"]))
    if c.get("v_scale") is not None:
        v = v * c["v_scale"].double()[:, :, None, None]
    v = torch.nan_to_num(v, nan=0.0)
    return vmax_valid(v, c["seq_lens"])


def run_case(lib, seed, B, Hq, Hkv, L, d, kv=torch.bfloat16, q_dtype=torch.float32, seq_lens=None,
             alibi=False, n_splits=0, k_scale=1.0):
    note("seed=%d B=%d Hq=%d Hkv=%d L=%d d=%d kv=%s q=%s lens=%s alibi=%s S=%d" %
         (seed, B, Hq, Hkv, L, d, kv, q_dtype, seq_lens, alibi, n_splits))
    c = W.random_case(seed, B, Hq, Hkv, L, d, q_dtype=q_dtype, kv_dtype=kv, seq_lens=seq_lens,
                      alibi=alibi, k_scale=k_scale)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"])
    out = gpu_decode(lib, c, n_splits)
    assert_parity(out, ref, kv, vmax_real(c), "seed=%d" % seed)
    return out, ref, c


# ----------------------------------------------------------------------------- small shapes

def test_gist_shape_31_keys_8_chunks(lib):
    """The gist's test: 31 keys, width 512, fp32, 8 chunks (seven of 4 keys, one of 3)."""
    run_case(lib, 100, 1, 1, 1, 31, 512, kv=torch.float32, n_splits=8)


@pytest.mark.parametrize("L,S", [(9, 8), (3, 8), (1, 4), (1, 1), (64, 64), (65, 64)])
def test_empty_and_tiny_chunks(lib, L, S):
    run_case(lib, 110 + L + S, 2, 4, 4, L, 128, n_splits=S)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("kv", [torch.float32, torch.bfloat16])
def test_head_dims_and_dtypes(lib, d, kv):
    """Several tiles per wave and a ragged last tile in every chunk (L=1000, S=3)."""
    run_case(lib, 120 + d, 2, 2, 2, 1000, d, kv=kv, n_splits=3)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 8, 31, 64, 255, 1024, 1025, 2000])
def test_split_count_sweep(lib, S):
    run_case(lib, 130, 1, 4, 4, 4099, 128, n_splits=S)


def test_ragged_lengths_with_poisoned_tail(lib):
    """Keys past each length are NaN; lengths include 0, 1, an odd size and the maximum."""
    lens = [0, 1, 777, 2048, 1500, 3]
    out, ref, c = run_case(lib, 140, 6, 8, 8, 2048, 128, seq_lens=lens, n_splits=5)
    assert (out[0] == 0).all()


@pytest.mark.parametrize("B,Hq,Hkv", [(100, 2, 2), (70, 8, 2), (130, 4, 4)])
def test_many_ragged_rows(lib, B, Hq, Hkv):
    """More batch rows than a wave has lanes, lengths from 0 to the maximum: the
    work-group -> (row, chunk) assignment that puts non-empty chunks first must still
    give every (row, head, chunk) partial exactly once."""
    g = torch.Generator().manual_seed(B + Hq)
    lens = torch.randint(0, 301, (B,), generator=g).tolist()
    lens[0], lens[-1], lens[B // 2] = 0, 300, 1
    run_case(lib, 145 + B, B, Hq, Hkv, 300, 64, seq_lens=lens, n_splits=5)


@pytest.mark.parametrize("g", [2, 4, 8])
def test_grouped_query_heads(lib, g):
    run_case(lib, 150 + g, 2, 4 * g, 4, 1500, 128, seq_lens=[1500, 913], n_splits=6)


def _repeat_heads(t, g):
    """Each KV head repeated g times along dim 1 (byte-wise, so FP8 tensors work too)."""
    if t is None:
        return None
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8).repeat_interleave(g, dim=1).contiguous().view(t.dtype)
    return t.repeat_interleave(g, dim=1).contiguous()


@pytest.mark.parametrize("kv,d,nq", [(torch.bfloat16, 128, 1), (torch.bfloat16, 64, 2),
                                     (torch.float8_e4m3fn, 128, 1)])
def test_gqa_equals_repeated_kv_mha(lib, kv, d, nq):
    """Grouped-query decoding equals multi-head decoding with every KV head repeated
    for its query group (the grouped and the one-head-per-work-group kernels, run on
    the same numbers)."""
    g, B, Hq, L = 4, 2, 32, 20000
    note("gqa vs repeated-kv mha kv=%s d=%d nq=%d" % (kv, d, nq))
    c = W.random_case(470 + d + nq, B, Hq, Hq // g, L, d, kv_dtype=kv, seq_lens=[L, 13457])
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(471))
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], k_scale=c["k_scale"],
                            v_scale=c["v_scale"])
    gqa = gpu_decode(lib, c, 0)
    mha_case = dict(c, k=_repeat_heads(c["k"], g), v=_repeat_heads(c["v"], g),
                    k_scale=_repeat_heads(c["k_scale"], g), v_scale=_repeat_heads(c["v_scale"], g))
    mha = gpu_decode(lib, mha_case, 0)
    vmax = vmax_real(c)
    assert_parity(gqa, ref, kv, vmax, "gqa")
    assert_parity(mha, ref, kv, vmax, "repeated-kv mha")
    assert np.abs(gqa - mha).max() <= 2e-3 * vmax


def test_alibi_bias(lib):
    run_case(lib, 160, 2, 16, 16, 3000, 128, seq_lens=[3000, 1234], alibi=True, n_splits=4)


def test_alibi_fp32_tight(lib):
    run_case(lib, 161, 1, 8, 8, 1000, 64, kv=torch.float32, alibi=True, n_splits=3)


def test_bf16_query(lib):
    run_case(lib, 170, 2, 4, 4, 700, 128, q_dtype=torch.bfloat16, n_splits=3)


def test_large_logits(lib):
    """K scaled by 6: logits span tens of units; the online max must keep exp() in range."""
    run_case(lib, 180, 1, 4, 4, 5000, 128, n_splits=7, k_scale=6.0)


def test_strided_and_3d_layouts(lib):
    """A [B, L, H, d] cache viewed as [B, H, L, d], and the 3-D [B, L, d] form."""
    c = W.random_case(190, 2, 4, 4, 600, 128)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"])
    kt = c["k"].transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    vt = c["v"].transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    out = lib.decode(c["q"].to(DEV), kt, vt, None, None, 5)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), ref, torch.bfloat16, vmax_valid(c["v"], None), "strided")
    c1 = W.random_case(191, 3, 1, 1, 500, 64)
    ref1 = oracle.decode_f64(c1["q"], c1["k"], c1["v"])
    out1 = lib.decode(c1["q"].to(DEV), c1["k"][:, 0].to(DEV), c1["v"][:, 0].to(DEV), None, None, 2)
    torch.cuda.synchronize()
    assert_parity(out1.cpu().numpy(), ref1, torch.bfloat16, vmax_valid(c1["v"], None), "3d")


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float32])
def test_entry_points_agree(lib, kv):
    """tad_decode (stream-ordered allocation), tad_decode_ws and tad_split + tad_combine
    give bit-identical outputs; repeated calls are bit-identical (fixed-order sums).
    bf16: grouped-query heads on the matrix cores (split + combine); fp32: the vector
    kernel with its fused merge (a small grid)."""
    c = to_dev(W.random_case(200, 2, 8, 2, 3333, 128, kv_dtype=kv, seq_lens=[3333, 2000], alibi=True))
    S = 6
    a = lib.decode(c["q"], c["k"], c["v"], c["seq_lens"], c["slopes"], S)
    out_b = torch.empty_like(a)
    lib.tad_decode(c["q"], c["k"], c["v"], c["seq_lens"], c["slopes"], S, out_b)
    ws = lib.workspace(c["q"], c["k"], S)
    lib.tad_split(c["q"], c["k"], c["v"], c["seq_lens"], c["slopes"], S, ws)
    out_c = torch.empty_like(a)
    lib.tad_combine(ws, 2, 8, 1, S, 128, out_c)
    again = lib.decode(c["q"], c["k"], c["v"], c["seq_lens"], c["slopes"], S)
    torch.cuda.synchronize()
    assert torch.equal(a, out_b) and torch.equal(a, out_c) and torch.equal(a, again)


FP8 = [torch.float8_e4m3fn, torch.float8_e5m2]


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("kv", FP8)
def test_fp8_head_dims(lib, d, kv):
    """OCP FP8 K/V with per-(b, head) dequantisation scales; several tiles and a ragged
    tail per chunk."""
    run_case(lib, 300 + d, 2, 2, 2, 1000, d, kv=kv, n_splits=3)


@pytest.mark.parametrize("kv", FP8)
def test_fp8_ragged_gqa_alibi(lib, kv):
    """FP8 with NaN bit patterns past each length, grouped heads and ALiBi."""
    run_case(lib, 310, 3, 8, 2, 3000, 128, kv=kv, seq_lens=[3000, 1, 2222], alibi=True, n_splits=4)


@pytest.mark.parametrize("kv", FP8)
@pytest.mark.parametrize("B,Hq,Hkv,d,nq,S", [
    (2, 8, 2, 128, 1, 5),        # 4 heads per KV head, one KV head per work-group
    (2, 32, 8, 128, 1, 3),       # few items: one KV head per work-group
    (3, 32, 8, 128, 1, 48),      # 4 KV heads per work-group (288 items), many chunks
    (2, 16, 4, 64, 1, 7),        # d 64
    (2, 8, 8, 128, 2, 64),       # several tokens, 4 KV heads per work-group (256 items)
    (3, 16, 4, 128, 3, 9),       # 4 heads x 3 tokens = 12 columns
    (2, 4, 4, 128, 16, 4),       # 16 tokens fill the 16 columns
    (3, 8, 4, 64, 4, 5),         # d 64, 2 heads x 4 tokens
    (2, 4, 2, 64, 3, 11),        # d 64, one KV head per work-group, several tokens
])
def test_fp8_matrix_core_path(lib, kv, B, Hq, Hkv, d, nq, S):
    """FP8 K/V with query-head groups or several tokens take the matrix-core kernel:
    32-key FP8 tiles, K operands and V^T (8-bit transposing read) widened to bf16 in
    registers, K scale folded into q, V scale into the partials.  Lengths include 1
    (shorter than the tokens: columns with no visible key) and ALiBi is on."""
    note("fp8 mfma kv=%s B=%d Hq=%d Hkv=%d d=%d nq=%d S=%d" % (kv, B, Hq, Hkv, d, nq, S))
    lens = [1700, 1, 999][:B]
    c = W.random_case(330 + Hkv + d + nq, B, Hq, Hkv, 1700, d, kv_dtype=kv, seq_lens=lens, alibi=True,
                      k_scale=3.0)
    if nq > 1:
        c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(331))
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"])
    out = gpu_decode(lib, c, S)
    assert_parity(out, ref, kv, vmax_real(c), "fp8 mfma")


def test_fp8_long_context(lib):
    run_case(lib, 320, 1, 8, 8, 65536, 128, kv=torch.float8_e4m3fn, n_splits=0, k_scale=4.0)


def multi_case(seed, B, Hq, Hkv, nq, L, d, kv=torch.bfloat16, lens=None, alibi=False):
    c = W.random_case(seed, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens, alibi=alibi)
    c["q"] = torch.randn((B, Hq, nq, d), generator=torch.Generator().manual_seed(seed + 9))
    return c


@pytest.mark.parametrize("B,Hq,Hkv,nq,kv,d", [
    (2, 4, 4, 2, torch.bfloat16, 128),      # matrix-core path: 2 tokens per head
    (1, 8, 8, 16, torch.bfloat16, 128),     # 16 tokens fill the 16 columns
    (2, 8, 2, 4, torch.bfloat16, 64),       # 4 heads x 4 tokens
    (2, 4, 4, 17, torch.bfloat16, 128),     # 17 columns: matrix cores, 2 column blocks
    (2, 8, 2, 5, torch.bfloat16, 128),      # 4 heads x 5 tokens: 2 column blocks
    (2, 4, 4, 3, torch.float32, 128),       # fp32: vector path
    (2, 4, 2, 3, torch.float8_e4m3fn, 256),
])
@pytest.mark.parametrize("alibi", [False, True])
def test_several_query_tokens(lib, B, Hq, Hkv, nq, kv, d, alibi):
    """nq new tokens per row, each seeing the keys up to its own position (causal among
    the new tokens); ragged lengths including one shorter than nq."""
    lens = [700, nq - 2][:B] if B > 1 else [1000]
    L = max(lens)
    note("tokens B=%d Hq=%d Hkv=%d nq=%d kv=%s d=%d alibi=%s lens=%s" % (B, Hq, Hkv, nq, kv, d, alibi, lens))
    c = multi_case(400 + nq + d, B, Hq, Hkv, nq, L, d, kv, lens, alibi)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], slopes=c["slopes"],
                            k_scale=c["k_scale"], v_scale=c["v_scale"])
    for S in (3, 40):
        out = gpu_decode(lib, c, S)
        assert out.shape == (B, Hq, nq, d)
        assert_parity(out, ref, kv, vmax_real(c), "tokens S=%d" % S)
    if B > 1:
        assert (out[1, :, :2] == 0).all()          # positions before the first key


def test_several_tokens_entry_points_agree(lib):
    """Fused (small) and split + combine give identical multi-token outputs."""
    c = to_dev(multi_case(450, 2, 8, 2, 3, 900, 128, lens=[900, 500]))
    S = 4
    a = lib.decode(c["q"], c["k"], c["v"], c["seq_lens"], None, S)
    ws = lib.workspace(c["q"], c["k"], S)
    lib.tad_split(c["q"], c["k"], c["v"], c["seq_lens"], None, S, ws)
    b = torch.empty_like(a)
    lib.tad_combine(ws, 2, 8, 3, S, 128, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv,nq", [(16, 4, 1), (32, 8, 1), (8, 8, 2)])
def test_grouped_kv_heads_decode_equals_split_combine(lib, Hq, Hkv, nq, d):
    """Grouped-query heads on the matrix cores, here a small grid at 3 chunks, where
    tad_decode_ws merges in the split kernel's last work-group per (row, KV head): it
    equals tad_split + tad_combine bit for bit, call after call, and is within the bar
    of the oracle."""
    note("grouped kv heads Hq=%d Hkv=%d nq=%d d=%d" % (Hq, Hkv, nq, d))
    c = W.random_case(460 + Hq + nq + d, 2, Hq, Hkv, 1800, d, seq_lens=[1800, 1001])
    if nq > 1:
        c["q"] = torch.randn((2, Hq, nq, d), generator=torch.Generator().manual_seed(461))
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"])
    g = to_dev(c)
    S = 3                                              # 2 * Hkv * 3 items <= CU count: fused
    a = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], None, S)
    again = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], None, S)
    ws = lib.workspace(g["q"], g["k"], S)
    lib.tad_split(g["q"], g["k"], g["v"], g["seq_lens"], None, S, ws)
    b = torch.empty_like(a)
    lib.tad_combine(ws, 2, Hq, nq, S, d, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, again)
    assert_parity(a.cpu().numpy(), ref, torch.bfloat16, vmax_real(c), "grouped kv heads")


def test_workspace_reuse_and_clear(lib):
    """On small grids tad_decode_ws merges in the vector split kernel's last work-group
    per row; its arrival counters return to zero, so one workspace serves call after
    call (and after tad_workspace_clear of a dirty buffer)."""
    c = to_dev(W.random_case(205, 2, 8, 8, 2500, 128, seq_lens=[2500, 1700]))
    c2 = to_dev(W.random_case(206, 2, 8, 8, 2500, 64))
    S = 5
    ref = lib.decode(c["q"], c["k"], c["v"], c["seq_lens"], None, S)
    ws = lib.workspace(c["q"], c["k"], S)
    outs = []
    for _ in range(4):
        out = torch.empty_like(ref)
        lib.tad_decode_ws(c["q"], c["k"], c["v"], c["seq_lens"], None, S, out, ws)
        outs.append(out)
    ws.fill_(0x5A)                                   # a dirty buffer, then an explicit clear
    lib.tad_workspace_clear(ws)
    out = torch.empty_like(ref)
    lib.tad_decode_ws(c["q"], c["k"], c["v"], c["seq_lens"], None, S, out, ws)
    outs.append(out)
    # a different problem (MHA, d 64) through a workspace of its own, twice
    ws2 = lib.workspace(c2["q"], c2["k"], 3)
    o2 = [torch.empty((2, 8, 64), device=DEV) for _ in range(2)]
    for o in o2:
        lib.tad_decode_ws(c2["q"], c2["k"], c2["v"], None, None, 3, o, ws2)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)
    assert torch.equal(o2[0], o2[1])
    ref2 = oracle.decode_f64(c2["q"].cpu(), c2["k"].cpu(), c2["v"].cpu())
    assert_parity(o2[0].cpu().numpy(), ref2, torch.bfloat16, vmax_valid(c2["v"].cpu(), None), "reuse d64")


# ----------------------------------------------------------------------------- partials

@pytest.mark.parametrize("alibi", [False, True])
def test_split_partials_match_chunk_statistics(lib, alibi):
    """tad_split's (m, l, o) equal the per-chunk (local_max, den, num) of the tree
    decoding steps, with m in base 2 (m * ln 2 = local_max)."""
    B, H, L, d, S = 1, 3, 2000, 128, 7
    c = W.random_case(210 + alibi, B, H, H, L, d, alibi=alibi)
    g = to_dev(c)
    m, l, o = lib.split_partials(g["q"], g["k"], g["v"], None, g["slopes"], S)
    torch.cuda.synchronize()
    m, l, o = m.cpu().double().numpy(), l.cpu().double().numpy(), o.cpu().double().numpy()
    for h in range(H):
        bias = None
        if alibi:
            bias = np.array([oracle.alibi_bias(L, j, float(c["slopes"][h])) for j in range(L)])
        parts = tree.chunk_partials(oracle.widen(c["q"])[0, h], oracle.widen(c["k"])[0, h],
                                    oracle.widen(c["v"])[0, h], S, bias)
        for s, (lm, den, num) in enumerate(parts):
            assert m[0, h, s] * math.log(2) == pytest.approx(lm, rel=1e-5, abs=1e-5)
            # rescale the GPU's l, o to the oracle's exact local max before comparing
            fix = math.exp(m[0, h, s] * math.log(2) - lm)
            assert l[0, h, s] * fix == pytest.approx(den, rel=1e-4)
            np.testing.assert_allclose(o[0, h, s] * fix, num, rtol=1e-4, atol=1e-4 * np.abs(num).max())


def test_split_partials_ragged_batch(lib):
    """With per-row lengths every row is cut with the batch-wide chunk length
    ceil(max L / S); shorter rows end in empty chunks."""
    lens = [2000, 700, 1333]
    B, H, L, d, S = 3, 2, 2000, 64, 7
    c = W.random_case(215, B, H, H, L, d, seq_lens=lens)
    g = to_dev(c)
    m, l, o = lib.split_partials(g["q"], g["k"], g["v"], g["seq_lens"], None, S)
    torch.cuda.synchronize()
    m, l, o = m.cpu().double().numpy(), l.cpu().double().numpy(), o.cpu().double().numpy()
    clen = -(-max(lens) // S)
    for b, Lb in enumerate(lens):
        for h in range(H):
            parts = tree.chunk_partials(oracle.widen(c["q"])[b, h], oracle.widen(c["k"])[b, h, :Lb],
                                        oracle.widen(c["v"])[b, h, :Lb], S, None, clen)
            for s, (lm, den, num) in enumerate(parts):
                if den == 0.0:
                    assert m[b, h, s] == -np.inf and l[b, h, s] == 0    # o is left unwritten
                    continue
                assert m[b, h, s] * math.log(2) == pytest.approx(lm, rel=1e-5, abs=1e-5)
                fix = math.exp(m[b, h, s] * math.log(2) - lm)
                assert l[b, h, s] * fix == pytest.approx(den, rel=1e-4)
                np.testing.assert_allclose(o[b, h, s] * fix, num, rtol=1e-4, atol=1e-4 * np.abs(num).max())


@pytest.mark.parametrize("B,Hq,Hkv,S", [(80, 16, 4, 5), (70, 32, 8, 3), (3, 32, 8, 64), (2, 8, 4, 12)])
def test_grouped_ragged_rows_busy_first(lib, B, Hq, Hkv, S):
    """Matrix-core kernel (4 KV heads per work-group from 256 items on): more rows than a
    wave has lanes, zero lengths and many empty chunks.  Work-group k serves the k-th chunk in
    busy-first order; every (row, head, chunk) partial must still be produced exactly
    once."""
    g = torch.Generator().manual_seed(B + S)
    L = 300 if B > 8 else 2000
    lens = torch.randint(0, L + 1, (B,), generator=g).tolist()
    lens[0], lens[-1], lens[B // 2] = 0, L, 1
    run_case(lib, 470 + B + S, B, Hq, Hkv, L, 128, seq_lens=lens, n_splits=S)


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float8_e4m3fn])
def test_grouped_split_partials_ragged(lib, kv):
    """Per-chunk partials of the matrix-core kernel on a ragged batch: the chunk
    statistics of the tree decoding steps, and the merge identity for empty chunks."""
    lens = [1500, 0, 333, 1100]
    B, Hq, Hkv, L, d, S = 4, 8, 4, 1500, 128, 9
    c = W.random_case(225, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens)
    g = to_dev(c)
    m, l, o = lib.split_partials(g["q"], g["k"], g["v"], g["seq_lens"], None, S, k_scale=g["k_scale"],
                                 v_scale=g["v_scale"])
    torch.cuda.synchronize()
    m, l, o = m.cpu().double().numpy(), l.cpu().double().numpy(), o.cpu().double().numpy()
    clen = -(-max(lens) // S)
    kw, vw = oracle.widen(c["k"]), oracle.widen(c["v"])
    if c["k_scale"] is not None:
        kw = kw * c["k_scale"].double().numpy()[:, :, None, None]
        vw = vw * c["v_scale"].double().numpy()[:, :, None, None]
    # q and the probabilities enter the matrix cores as two bf16 terms each (hi + lo,
    # both truncations: |x - hi - lo| < 2^-14 |x|, and about 2^-16 |x| on average), K
    # and V exactly; accumulation is fp32.  Each score is then off by at most
    # 2^-14 sum_i |q_i k_i| (a few 1e-4 here) but by ~1e-5 typically, with signs that
    # average out over a chunk's keys, and each weight by 2^-14 at most.  The bar
    # 2.5e-4 (relative for l, relative to the chunk's largest |o| for o) is 10x above
    # the typical error yet below what dropping either lo term gives (q lo: ~4e-3 per
    # weight, ~1e-3 on o; P lo: a one-sided truncation bias of ~2e-3 on o).
    tol = 2.5e-4
    worst_l = worst_o = 0.0
    for b, Lb in enumerate(lens):
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            parts = tree.chunk_partials(oracle.widen(c["q"])[b, h], kw[b, kh, :Lb], vw[b, kh, :Lb], S, None, clen)
            for s, (lm, den, num) in enumerate(parts):
                if den == 0.0:
                    assert m[b, h, s] == -np.inf and l[b, h, s] == 0    # o is left unwritten
                    continue
                assert m[b, h, s] * math.log(2) == pytest.approx(lm, rel=1e-4, abs=1e-4)
                fix = math.exp(m[b, h, s] * math.log(2) - lm)
                worst_l = max(worst_l, abs(l[b, h, s] * fix / den - 1))
                worst_o = max(worst_o, float(np.abs(o[b, h, s] * fix - num).max() / np.abs(num).max()))
                assert l[b, h, s] * fix == pytest.approx(den, rel=tol)
                np.testing.assert_allclose(o[b, h, s] * fix, num, rtol=tol, atol=tol * np.abs(num).max())
    note("matrix-core partials kv=%s: worst relative error l %.2e, o %.2e (bar %.1e)" % (kv, worst_l, worst_o, tol))


@pytest.mark.parametrize("B,Hq,Hkv,L,d,kv,S", [
    (1100, 4, 2, 64, 128, torch.bfloat16, 2),      # one KV head per work-group
    (300, 16, 4, 40, 128, torch.bfloat16, 2),      # 4 KV heads per work-group, d 128
    (600, 16, 4, 48, 64, torch.float8_e4m3fn, 3),  # 4 KV heads per work-group, d 64, FP8
])
def test_more_busy_items_than_work_groups(lib, B, Hq, Hkv, L, d, kv, S):
    """The matrix-core grid holds at most one work-group per resident slot.  With more
    (row, KV-head group) pairs than slots even the longest chunk length leaves more
    busy items than work-groups, and work-groups run several busy items in turn."""
    g = torch.Generator().manual_seed(B + d)
    lens = torch.randint(0, L + 1, (B,), generator=g).tolist()
    lens[0], lens[-1], lens[B // 2] = 0, L, 1
    run_case(lib, 480 + B + d, B, Hq, Hkv, L, d, kv=kv, seq_lens=lens, n_splits=S)


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float8_e4m3fn])
def test_empty_items_beyond_the_grid(lib, kv):
    """Many more chunks than resident work-groups on a ragged batch: the empty chunks
    are written by work-groups that already ran a busy one.  The workspace starts as
    NaN, so every (row, head, chunk) m and l must be written, and the o of every
    non-empty chunk (an empty chunk's o stays NaN and the merge must ignore it); the
    merge matches the oracle."""
    B, Hq, Hkv, L, d, S = 8, 32, 8, 3000, 128, 96
    lens = [3000, 17, 0, 1204, 2999, 300, 1, 2048]
    note("empty items beyond the grid kv=%s S=%d" % (kv, S))
    c = W.random_case(490, B, Hq, Hkv, L, d, kv_dtype=kv, seq_lens=lens)
    ref = oracle.decode_f64(c["q"], c["k"], c["v"], seq_lens=c["seq_lens"], k_scale=c["k_scale"],
                            v_scale=c["v_scale"])
    gd = to_dev(c)
    ws = lib.workspace(gd["q"], gd["k"], S)
    n = B * Hq * S
    al = lambda x: (x + 255) // 256 * 256
    mlo = ws[:al(4 * n) * 2 + 4 * n * d].view(torch.float32)
    mlo.fill_(float("nan"))
    lib.tad_split(gd["q"], gd["k"], gd["v"], gd["seq_lens"], None, S, ws, None, gd["k_scale"], gd["v_scale"])
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    lib.tad_combine(ws, B, Hq, 1, S, d, out)
    torch.cuda.synchronize()
    m, l = mlo[:n], mlo[al(4 * n) // 4:al(4 * n) // 4 + n]
    o = mlo[2 * al(4 * n) // 4:].view(n, d)
    assert not torch.isnan(m).any() and not torch.isnan(l).any()
    assert not torch.isnan(o[torch.isfinite(m)]).any()      # o of every non-empty chunk
    assert (l[torch.isinf(m)] == 0).all()
    assert_parity(out.cpu().numpy(), ref, kv, vmax_real(c), "empty items")


def test_empty_chunk_partials(lib):
    """Chunks past the sequence end are the merge identity: m = -inf, l = 0 (their o
    is not part of the result: the merge gives them weight 0)."""
    c = to_dev(W.random_case(220, 1, 2, 2, 9, 64))
    m, l, o = lib.split_partials(c["q"], c["k"], c["v"], None, None, 8)
    torch.cuda.synchronize()
    # 9 keys over 8 chunks: length 2, chunks 5..7 empty
    assert torch.isinf(m[:, :, 5:]).all() and (m[:, :, 5:] < 0).all()
    assert (l[:, :, 5:] == 0).all()
    assert torch.isfinite(m[:, :, :5]).all()


# ----------------------------------------------------------------------------- invariants

def test_zero_query_is_mean(lib):
    c = W.random_case(230, 1, 4, 4, 10000, 128)
    c["q"].zero_()
    out = gpu_decode(lib, c, 9)
    mean = oracle.widen(c["v"]).mean(axis=2)
    assert np.abs(out - mean).max() <= 2e-6


def test_dominant_key_and_value_shift(lib):
    """O(1)-magnitude pins at long context: a planted key returns its V row; V + c
    shifts the output by c."""
    B, H, L, d = 1, 4, 50000, 128
    q = W.draw_q(240, B, H, d)
    k = W.draw_kv(241, B, H, L, d, torch.bfloat16)
    v = W.draw_kv(242, B, H, L, d, torch.bfloat16)
    pos = W.plant_dominant_keys(243, q, k, 60.0)
    out = gpu_decode(lib, dict(q=q, k=k, v=v, seq_lens=None, slopes=None), 0)
    for h in range(H):
        np.testing.assert_allclose(out[0, h], oracle.widen(v)[0, h, int(pos[0, h])], atol=1e-5)
    c = W.random_case(244, 1, 4, 4, 50000, 128)
    base = gpu_decode(lib, c, 0)
    c["v"] = (c["v"].float() + 2.0).to(torch.bfloat16)
    ref2 = oracle.decode_f64(c["q"], c["k"], c["v"])
    shifted = gpu_decode(lib, c, 0)
    assert_parity(shifted, ref2, torch.bfloat16, vmax_valid(c["v"], None), "v+2")
    assert np.abs(shifted.mean() - base.mean() - 2.0) < 1e-2


@pytest.mark.parametrize("B,Hq,Hkv,nq,Lmax,d,kv", [
    (1, 32, 32, 1, 131072, 128, torch.bfloat16), (8, 32, 8, 1, 32768, 128, torch.bfloat16),
    (8, 32, 8, 1, 32768, 128, torch.float8_e4m3fn), (4, 16, 16, 1, 65536, 128, torch.bfloat16),
    (1, 8, 8, 1, 1 << 20, 128, torch.bfloat16), (1, 1, 1, 1, 4096, 512, torch.float32),
    (2, 1, 1, 1, 300, 64, torch.bfloat16), (64, 32, 32, 1, 4096, 128, torch.bfloat16),
    (1, 1, 1, 1, 100, 128, torch.float32), (1, 32, 32, 1, 1024, 128, torch.bfloat16),
    (2, 16, 2, 1, 16384, 128, torch.float8_e5m2), (1, 32, 8, 1, 4096, 128, torch.bfloat16),
    (1, 8, 8, 2, 4096, 64, torch.bfloat16), (1, 32, 8, 1, 4096, 256, torch.bfloat16),
    (1, 128, 8, 2, 4096, 128, torch.bfloat16)])
def test_auto_splits_rule(lib, B, Hq, Hkv, nq, Lmax, d, kv):
    """The documented automatic chunk count: ceil(4 CUs / (B Hkv)) for one row,
    ceil(6 CUs / (B Hkv)) for several, no work-group chunk under 128 KiB of K and V
    (32 KiB per KV head where the matrix-core kernel takes 4 KV heads per work-group),
    at least 1."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per_cu = 4 if B == 1 else 6
    elem = torch.empty((), dtype=kv).element_size()
    gq = Hq // Hkv * nq
    matrix = d in (64, 128, 256) and kv != torch.float32 and 2 <= gq <= 256
    heads_per_wg = 4 if matrix and Hkv % 4 == 0 and (gq <= 16 or d == 256) else 1
    want = max(1, min(-(-per_cu * cus // (B * Hkv)), Lmax * 2 * d * elem * heads_per_wg // (128 << 10), 4096))
    assert lib.tad_auto_splits(B, Hq, Hkv, nq, Lmax, d, kv, 0) == want


@pytest.mark.parametrize("d,kv,L", [(512, torch.float32, 4096), (256, torch.bfloat16, 6000)])
@pytest.mark.parametrize("S", [8, 64, 256, 0])
def test_one_head_many_chunks(lib, d, kv, L, S):
    """One head cut into many chunks (the automatic count gives a single fp32 d = 512
    head of 4096 keys 128 of them): the combine spreads the row's columns over
    work-groups, each column summed by several thread rows; S = 8 merges in the split
    kernel's last work-group instead."""
    run_case(lib, 500 + d + S, 1, 1, 1, L, d, kv=kv, n_splits=S)


@pytest.mark.parametrize("d", [64, 256, 512])
def test_fused_merge_equals_combine_wide_heads(lib, d):
    """The fused merge (small grid, <= 8 chunks) and the combine kernel run the same
    fixed-order merge, also where a row's columns form several groups: tad_decode_ws
    equals tad_split + tad_combine bit for bit."""
    c = to_dev(W.random_case(510 + d, 1, 2, 2, 2500, d, kv_dtype=torch.float32, seq_lens=[1999]))
    S = 7
    ws = lib.workspace(c["q"], c["k"], S)
    a = torch.empty((1, 2, d), dtype=torch.float32, device=DEV)
    lib.tad_decode_ws(c["q"], c["k"], c["v"], c["seq_lens"], None, S, a, ws)
    ws2 = lib.workspace(c["q"], c["k"], S)
    lib.tad_split(c["q"], c["k"], c["v"], c["seq_lens"], None, S, ws2)
    b = torch.empty_like(a)
    lib.tad_combine(ws2, 1, 2, 1, S, d, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.decode_f64(c["q"].cpu(), c["k"].cpu(), c["v"].cpu(), seq_lens=c["seq_lens"].cpu())
    assert_parity(a.cpu().numpy(), ref, torch.float32, 0.0, "fused d=%d" % d)
