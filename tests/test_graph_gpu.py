"""The allocation-free entry points inside a captured HIP graph.

tad_decode_ws and tad_decode_paged_ws launch only kernels (no allocation, no memset),
so a caller may capture them.  Each case captures one call, then replays the graph
several times with eager work (and a new query written into the captured buffer)
between replays; every replay must equal the eager call bit for bit.
"""
import pytest
import torch

import workloads as W
from test_parity_gpu import DEV

pytestmark = pytest.mark.gpu


def dev(x):
    return None if x is None else x.to(DEV)


@pytest.mark.parametrize("case", ["fused-mha", "gqa", "split-combine-mha", "paged-interleaved", "tokens",
                                  "gqa-many-chunks", "pieces", "pieces-combine", "fp8-block-gqa",
                                  "fp8-block-split-combine", "wide-columns", "d256-fused", "d256-many-chunks",
                                  "combine-scan"])
def test_decode_ws_replays_in_a_graph(lib, case):
    print("[case] graph %s" % case, flush=True)
    paged = case == "paged-interleaved"
    if case == "fused-mha":           # small grid: one launch, merge in the last work-group
        c, S = W.random_case(900, 2, 8, 8, 2500, 128, seq_lens=[2500, 1700]), 5
    elif case == "gqa":               # matrix-core split, merge in its last work-group per KV head
        c, S = W.random_case(906, 2, 8, 2, 2500, 128, seq_lens=[2500, 1700]), 5
    elif case == "split-combine-mha":  # large grid: split then combine
        c, S = W.random_case(901, 2, 32, 32, 4000, 128, seq_lens=[4000, 3333]), 16
    elif case == "gqa-many-chunks":   # more chunks than resident work-groups: waves write empty chunks
        c, S = W.random_case(907, 8, 32, 8, 3000, 128, seq_lens=[3000, 17, 0, 1204, 2999, 300, 1, 2048]), 96
    elif case == "pieces":            # one head, 8 chunks read as pieces, then the fused row merge
        c, S = W.random_case(908, 1, 1, 1, 4096, 512, kv_dtype=torch.float32), 8
    elif case == "pieces-combine":    # 40 chunks read as pieces, then the combine kernel
        c, S = W.random_case(909, 1, 2, 2, 60000, 128), 40
    elif case == "fp8-block-gqa":     # FP8 with 32-key scale blocks, matrix-core one-launch form
        c, S = W.random_case(910, 2, 8, 2, 2500, 128, kv_dtype=torch.float8_e4m3fn, seq_lens=[2500, 1700],
                             scale_block=32), 5
    elif case == "fp8-block-split-combine":   # FP8 with 64-key scale blocks, vector split then combine
        c, S = W.random_case(911, 2, 32, 32, 4000, 128, kv_dtype=torch.float8_e5m2, seq_lens=[4000, 3333],
                             scale_block=64), 16
    elif case == "wide-columns":      # 8 heads x 4 tokens = 32 columns per KV head: two blocks per wave
        c, S = W.random_case(912, 2, 8, 1, 2000, 128, seq_lens=[2000, 900]), 6
        c["q"] = torch.randn((2, 8, 4, 128), generator=torch.Generator().manual_seed(915))
    elif case == "d256-fused":        # d 256 on the matrix cores, merge in its last work-group per KV head
        c, S = W.random_case(913, 2, 8, 4, 1500, 256, seq_lens=[1500, 800]), 4
    elif case == "d256-many-chunks":  # d 256, 4 KV heads per work-group, more chunks than resident work-groups
        c, S = W.random_case(914, 8, 16, 8, 2000, 256, seq_lens=[2000, 17, 0, 1204, 1999, 300, 1, 1024]), 96
    elif case == "combine-scan":      # 2048 (head, token) rows x 24 chunks: the combine reads m first
        c, S = W.random_case(916, 8, 32, 8, 4000, 128, seq_lens=[4000, 17, 0, 1204, 3999, 300, 1, 2048]), 24
        c["q"] = torch.randn((8, 32, 8, 128), generator=torch.Generator().manual_seed(917))
    elif case == "tokens":
        c, S = W.random_case(902, 2, 8, 2, 1500, 128, seq_lens=[1500, 900]), 6
        c["q"] = torch.randn((2, 8, 3, 128), generator=torch.Generator().manual_seed(903))
    else:                             # token-major pages: head-packed split, merge in its last work-groups
        c, S = W.random_case(904, 2, 16, 16, 2000, 128, seq_lens=[2000, 1111]), 8
    q, k, v, sl = dev(c["q"]), dev(c["k"]), dev(c["v"]), dev(c["seq_lens"])
    blk = {"fp8-block-gqa": 32, "fp8-block-split-combine": 64}.get(case, 0)
    kw = dict(k_scale=dev(c["k_scale"]), v_scale=dev(c["v_scale"]), k_scale_block=blk, v_scale_block=blk)
    if paged:
        kc, vc, tb = W.page_kv(c["k"], c["v"], 16, 904)
        kc, vc, tb = dev(kc), dev(vc), dev(tb)

    def call(out, ws):
        if paged:
            lib.tad_decode_paged_ws(q, kc, vc, tb, sl, None, S, out, ws)
        else:
            lib.tad_decode_ws(q, k, v, sl, None, S, out, ws, **kw)

    def eager():
        out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        ws = lib.workspace(q, k, S)
        call(out, ws)
        torch.cuda.synchronize()
        return out

    ref = eager()
    out = torch.empty_like(ref)
    ws = lib.workspace(q, k, S)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up call off the capture
        call(out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, ws)
    n_part = q.shape[0] * q.shape[1] * (q.shape[2] if q.dim() == 4 else 1) * S
    al = lambda x: (x + 255) // 256 * 256
    partials = ws[:2 * al(4 * n_part) + 4 * n_part * q.shape[-1]].view(torch.float32)
    for i in range(3):
        out.fill_(float("nan"))                       # eager work between replays
        if case in ("gqa-many-chunks", "d256-many-chunks", "combine-scan"):
            partials.fill_(float("nan"))              # every partial must be written again
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d" % i
    # a new query written into the captured buffer: the replay decodes it
    q.copy_(torch.randn(q.shape, generator=torch.Generator().manual_seed(905)).to(DEV))
    ref2 = eager()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2)
    assert not torch.equal(ref, ref2)
