"""GPU: the combine kernel's two forms on the same partials.

tad_combine merges a call's chunk partials (m in base 2, l, o) with the global max /
renormalise / sum / divide of tree_attn_decode ("Tree Attention Decoding").  Calls
with at most 64 chunks and at least 1024 (head, token) rows merge 4 rows per
work-group; others spread each row's columns over work-groups.  Both keep one
summation order, so a row must come out with the same bits either way, and within
fp32 rounding of the merge computed in fp64 from the partials.
"""
import numpy as np
import pytest
import torch

from test_parity_gpu import DEV, note

pytestmark = pytest.mark.gpu


def layout(rows, S, d):
    al = lambda x: (x + 255) // 256 * 256
    n = rows * S
    return 0, al(4 * n), 2 * al(4 * n), n


def fill_partials(lib, rows_shape, S, d, seed, tail=0):
    """A workspace for B x Hq x nq rows holding seeded partials: maxima spread over 40
    (base 2), some empty chunks (m = -inf, l = 0, o left as garbage), one row empty;
    with tail > 0 the rows of even batch rows end with `tail` empty chunks (as a ragged
    batch's shorter rows do)."""
    B, Hq, nq = rows_shape
    rows = B * Hq * nq
    q = torch.zeros((B, Hq, nq, d), device=DEV)
    k = torch.zeros((B, 1, 16, d), dtype=torch.bfloat16, device=DEV)
    ws = lib.workspace(q, k, S)
    g = torch.Generator().manual_seed(seed)
    m = torch.randn((rows, S), generator=g, dtype=torch.float64) * 10
    l = torch.rand((rows, S), generator=g, dtype=torch.float64) * 50 + 1
    o = torch.randn((rows, S, d), generator=g, dtype=torch.float64) * 20
    empty = torch.rand((rows, S), generator=g) < 0.25
    empty[3] = True                                   # a row with no keys at all
    if tail:
        per_b = Hq * nq
        for b in range(0, B, 2):
            empty[b * per_b:(b + 1) * per_b, S - tail:] = True
    m[empty] = -np.inf
    l[empty] = 0.0
    o[empty] = float("nan")                           # never read with weight 0
    om, ol, oo, n = layout(rows, S, d)
    ws[om:om + 4 * n].view(torch.float32).copy_(m.float().flatten())
    ws[ol:ol + 4 * n].view(torch.float32).copy_(l.float().flatten())
    ws[oo:oo + 4 * n * d].view(torch.float32).copy_(o.float().flatten())
    return ws, m.float().double(), l.float().double(), o.float().double()


def merge_f64(m, l, o):
    """The merge of each row's chunk partials in fp64 (weights 2^(m_s - M))."""
    M = m.max(dim=1, keepdim=True).values
    M = torch.where(torch.isinf(M), torch.zeros_like(M), M)
    w = torch.exp2(m - M)
    w = torch.where(torch.isinf(m), torch.zeros_like(w), w)
    L = (w * l).sum(dim=1)
    O = torch.nan_to_num(w[:, :, None] * o, nan=0.0).sum(dim=1)
    return torch.where(L[:, None] > 0, O / L[:, None], torch.zeros_like(O))


@pytest.mark.parametrize("d,S,nq,tail", [(128, 24, 4, 0), (64, 64, 2, 0), (256, 7, 1, 0), (128, 1, 8, 0),
                                         (128, 48, 8, 10), (64, 64, 4, 63)])
def test_row_batched_combine_matches_column_split(lib, d, S, nq, tail):
    """The last two cases hold 16 MB of o partials or more, where the combine first reads
    the rows' m and skips the o of chunks past the last non-empty one; their trailing
    empty chunks hold NaN o, which must not be read with a nonzero weight."""
    B, Hq = 1024 // (31 * nq) + 1, 31                  # more than 1024 rows (not a multiple of 4 for nq < 4)
    rows = B * Hq * nq
    note("combine rows=%d S=%d d=%d tail=%d" % (rows, S, d, tail))
    ws, m, l, o = fill_partials(lib, (B, Hq, nq), S, d, 40 + S + d, tail)
    big = torch.empty((B, Hq, nq, d), dtype=torch.float32, device=DEV)
    lib.tad_combine(ws, B, Hq, nq, S, d, big)
    # the first batch row alone (Hq * nq < 1024 rows): the column-split form
    ws1, _, _, _ = fill_partials(lib, (1, Hq, nq), S, d, 40 + S + d, tail)
    om, ol, oo, n = layout(rows, S, d)
    om1, ol1, oo1, n1 = layout(Hq * nq, S, d)
    ws1[om1:om1 + 4 * n1].copy_(ws[om:om + 4 * n1])
    ws1[ol1:ol1 + 4 * n1].copy_(ws[ol:ol + 4 * n1])
    ws1[oo1:oo1 + 4 * n1 * d].copy_(ws[oo:oo + 4 * n1 * d])
    small = torch.empty((1, Hq, nq, d), dtype=torch.float32, device=DEV)
    lib.tad_combine(ws1, 1, Hq, nq, S, d, small)
    torch.cuda.synchronize()
    assert torch.equal(big[:1], small)
    ref = merge_f64(m, l, o).view(B, Hq, nq, d)
    got = big.double().cpu()
    assert torch.isfinite(got).all()
    assert (got.reshape(rows, d)[3] == 0).all()
    err = (got - ref).abs().max().item()
    assert err <= 1e-5 * max(1.0, ref.abs().max().item()), err
