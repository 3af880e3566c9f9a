"""GPU parity of grouped-query decode at head dimension 256 on the matrix cores.

At d = 256 a wave's q operands (hi + lo) and O take twice d = 128's registers, so the
kernel runs one wave per SIMD (its accumulators partly in AGPRs): one KV head per
4-wave work-group, or 4 KV heads of one wave each.  Against the fp64 oracle under the
usual bars; the small-grid one-launch form bit-identical to tad_split + tad_combine;
cases cover bf16 and FP8 K/V (per-head and per-block scales), several tokens (with
more than 16 columns per KV head: one 16-column block per work-group), ALiBi, ragged
rows with zeros, a paged cache, and 4 KV heads per work-group.
"""
import pytest
import torch

import oracle
import workloads as W
from test_column_blocks_gpu import oracle_ref, split_combine_poisoned, tokens_case, vmax_of
from test_paged_gpu import oracle_of, paged_case, run_paged
from test_parity_gpu import assert_parity, note, to_dev, vmax_real

pytestmark = pytest.mark.gpu

BF16, E4M3, E5M2 = torch.bfloat16, torch.float8_e4m3fn, torch.float8_e5m2


@pytest.mark.parametrize("B,Hq,Hkv,nq,kv,lens,S,alibi,blk", [
    (2, 8, 4, 1, BF16, [1500, 700], 5, False, 0),          # one launch (small grid), g 2
    (2, 16, 8, 1, BF16, [3000, 0], 200, True, 0),           # 4 KV heads per work-group, an empty row
    (3, 8, 2, 3, E4M3, [900, 1, 1300], 12, False, 0),       # FP8, 4 heads x 3 tokens, a row shorter than nq
    (2, 8, 1, 4, BF16, [1000, 600], 6, True, 0),            # 32 columns: two blocks, a work-group each
    (2, 8, 4, 2, E5M2, [2000, 1234], 7, False, 64),         # FP8 with 64-key scale blocks
    (1, 4, 2, 1, E5M2, [3000], 0, False, 0),                # automatic chunks
    (8, 32, 8, 1, BF16, "random", 24, False, 0),            # ragged batch, 4 KV heads per work-group
])
def test_d256_grouped_query(lib, B, Hq, Hkv, nq, kv, lens, S, alibi, blk):
    d = 256
    if lens == "random":
        lens = torch.randint(0, 4001, (B,), generator=torch.Generator().manual_seed(1234)).tolist()
        lens[0] = 4000
    note("d256 B=%d Hq=%d Hkv=%d nq=%d kv=%s lens=%s S=%d alibi=%s blk=%d" % (B, Hq, Hkv, nq, kv, lens, S,
                                                                            alibi, blk))
    c = tokens_case(1300 + B + Hq + nq + S, B, Hq, Hkv, nq, max(lens), d, kv, lens, alibi, blk)
    ref = oracle_ref(c, blk)
    g = to_dev(c)
    SS = lib.resolve_splits(g["q"], g["k"], S)
    a = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], SS, k_scale=g.get("k_scale"),
                   v_scale=g.get("v_scale"), k_scale_block=blk, v_scale_block=blk)
    again = lib.decode(g["q"], g["k"], g["v"], g["seq_lens"], g["slopes"], SS, k_scale=g.get("k_scale"),
                       v_scale=g.get("v_scale"), k_scale_block=blk, v_scale_block=blk)
    b = split_combine_poisoned(lib, g, SS, blk)
    torch.cuda.synchronize()
    assert torch.equal(a, again) and torch.equal(a, b)
    assert_parity(a.cpu().numpy(), ref, kv, vmax_of(c, blk), "d256")


@pytest.mark.parametrize("ps,kv,nq", [(16, BF16, 1), (32, E4M3, 2)])
def test_d256_paged(lib, ps, kv, nq):
    """Paged cache of d = 256 rows, 2 query heads per KV head."""
    note("d256 paged ps=%d kv=%s nq=%d" % (ps, kv, nq))
    c = paged_case(1350 + ps + nq, 2, 8, 4, 1200, 256, ps, kv, lens=[1200, 333], alibi=True, nq=nq)
    ref = oracle_of(c)
    for S in (3, 0):
        assert_parity(run_paged(lib, c, S), ref, kv, vmax_real(c), "d256 paged S=%d" % S)
