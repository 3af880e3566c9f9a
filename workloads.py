"""Seeded synthetic inputs for single-query attention decoding.

This module only draws random numbers and lays them out; it holds none of the
decoding arithmetic, so both the fp64 CPU oracle (under ``oracle/``) and the GPU
path may take their inputs from it without sharing any of the method.

Every tensor comes from its own ``torch.Generator`` on the CPU, seeded
``1000 * workload_id + t`` with t = 0 (q), 1 (K), 2 (V), 3 (sequence lengths),
4 (planted positions).  fp32 values are N(0, 1) from ``torch.randn``; bf16
tensors are those fp32 draws rounded to nearest-even by ``Tensor.to``.  K and V
are drawn one (batch, kv-head) slab at a time, in row-major order, so host
memory stays bounded for the long-context workloads.

Workloads (sizes as used by the tests and the benchmark):

=====  =========================================================================
id     description
=====  =========================================================================
1      single head, fp32: q [1,1,512]; K, V [1,4096,512] N(0,1); 8 equal chunks;
       no bias.  (The tree-attention gist's test shape with a longer sequence.)
2      MHA: batch 1, 32 heads, d 128, 131072 keys; q fp32, K/V bf16; split
       count chosen automatically.
3      GQA: batch 8, 32 query heads over 8 KV heads, d 128, K/V bf16; per-batch
       lengths uniform on [1024, 32768] (inclusive) in a [8,8,32768,128] cache;
       keys past each length are NaN.
4      ALiBi: batch 4, 16 heads, d 128, 65536 keys, K/V bf16; slope of head h is
       2^(-8(h+1)/16); only the slopes are passed.
5      1M-key stress: batch 1, 8 heads, d 128, 1048576 keys, K/V bf16; K is
       bf16(6 N(0,1)); one key per head, at a seeded position, is replaced by
       bf16(c q_h) with c = 60 sqrt(d) / |q_h|^2 so that its logit is about +60.
6      workload 2 with FP8 (OCP E4M3) K and V: each (b, kv-head) slab of N(0,1)
       draws is divided by its amax/448 and rounded to E4M3; the scale is kept.
7      workload 3 with FP8 (OCP E4M3) K and V, quantised as in workload 6; keys
       past each length hold the E4M3 NaN pattern.
=====  =========================================================================

``page_kv`` lays any of these K/V tensors out as a paged cache: pages of
``page_size`` rows in a pool with a few spare pages, assigned to (b, logical page)
by a seeded random permutation (seed + 5), every unused row poisoned with NaN.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

F32 = torch.float32
BF16 = torch.bfloat16


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    Lmax: int
    q_dtype: torch.dtype
    kv_dtype: torch.dtype
    n_splits: int = 0          # <= 0: automatic
    ragged: bool = False       # per-batch lengths on [ragged_lo, Lmax]
    ragged_lo: int = 1024
    alibi: bool = False
    k_scale: float = 1.0
    planted_logit: Optional[float] = None

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def kv_bytes(self, seq_lens: Optional[torch.Tensor] = None) -> int:
        """Algorithmic K+V bytes one decode reads: 2 * d * elem * keys per KV head."""
        elem = 4 if self.kv_dtype == F32 else (1 if self.kv_dtype in FP8_MAX else 2)
        if seq_lens is None:
            keys = self.B * self.Lmax
        else:
            keys = int(seq_lens.clamp(0, self.Lmax).sum().item())
        return 2 * self.d * elem * keys * self.Hkv


WORKLOADS = {
    1: Workload(1, "single-head fp32 d512 L4096 8 chunks", 1, 1, 1, 512, 4096, F32, F32, n_splits=8),
    2: Workload(2, "MHA B1 H32 d128 L131072 bf16", 1, 32, 32, 128, 131072, F32, BF16),
    3: Workload(3, "GQA B8 Hq32 Hkv8 d128 ragged L<=32768 bf16", 8, 32, 8, 128, 32768, F32, BF16,
                ragged=True),
    4: Workload(4, "ALiBi B4 H16 d128 L65536 bf16", 4, 16, 16, 128, 65536, F32, BF16, alibi=True),
    5: Workload(5, "1M-key stress B1 H8 d128 L1048576 bf16, planted key", 1, 8, 8, 128, 1 << 20,
                F32, BF16, k_scale=6.0, planted_logit=60.0),
    6: Workload(6, "MHA B1 H32 d128 L131072 fp8-e4m3 K/V, per-head scales", 1, 32, 32, 128, 131072,
                F32, torch.float8_e4m3fn),
    7: Workload(7, "GQA B8 Hq32 Hkv8 d128 ragged L<=32768 fp8-e4m3 K/V, per-head scales", 8, 32, 8, 128, 32768,
                F32, torch.float8_e4m3fn, ragged=True),
}


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(seed)


def alibi_slopes(H: int) -> torch.Tensor:
    """Per-head ALiBi slopes 2^(-8(h+1)/H), h = 0..H-1, as fp32."""
    h = torch.arange(1, H + 1, dtype=torch.float64)
    return torch.pow(2.0, -8.0 * h / H).to(F32)


def draw_q(seed: int, B: int, Hq: int, d: int, dtype=F32) -> torch.Tensor:
    q = torch.randn((B, Hq, d), generator=_gen(seed), dtype=F32)
    return q.to(dtype)


def draw_kv(seed: int, B: int, Hkv: int, L: int, d: int, dtype=BF16, scale: float = 1.0,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[B, Hkv, L, d] N(0,1)*scale drawn slab by slab (one (b, h) at a time)."""
    g = _gen(seed)
    if out is None:
        out = torch.empty((B, Hkv, L, d), dtype=dtype)
    for b in range(B):
        for h in range(Hkv):
            slab = torch.randn((L, d), generator=g, dtype=F32)
            if scale != 1.0:
                slab.mul_(scale)
            out[b, h].copy_(slab.to(dtype))
    return out


FP8_MAX = {torch.float8_e4m3fn: 448.0, torch.float8_e5m2: 57344.0}


def draw_kv_fp8(seed: int, B: int, Hkv: int, L: int, d: int, dtype=torch.float8_e4m3fn):
    """N(0,1) K or V quantised to FP8 with one scale per (b, kv-head) slab.

    The slab's scale is amax / (largest finite value of the format); the stored value is
    the N(0,1) draw divided by the scale, rounded by Tensor.to.  Returns (stored
    [B, Hkv, L, d] fp8, scales [B, Hkv] fp32) -- real value = stored * scale."""
    g = _gen(seed)
    out = torch.empty((B, Hkv, L, d), dtype=dtype)
    scale = torch.empty((B, Hkv), dtype=F32)
    for b in range(B):
        for h in range(Hkv):
            slab = torch.randn((L, d), generator=g, dtype=F32)
            s = float(slab.abs().max()) / FP8_MAX[dtype]
            scale[b, h] = s
            out[b, h].copy_((slab / scale[b, h]).to(dtype))
    return out, scale


def draw_kv_fp8_blocks(seed: int, B: int, Hkv: int, L: int, d: int, block: int, dtype=torch.float8_e4m3fn):
    """N(0,1) K or V quantised to FP8 with one scale per (b, kv-head, block of ``block`` keys).

    Each block's rows are N(0,1) draws times a seeded amplitude 2^u, u uniform on
    [-2, 2] (so neighbouring blocks differ in range), divided by the block's
    amax / (largest finite value of the format) and rounded by Tensor.to.  Returns
    (stored [B, Hkv, L, d] fp8, scales [B, Hkv, ceil(L / block)] fp32) -- key j's real
    value is stored * scale[..., j // block]."""
    g = _gen(seed)
    nblk = (L + block - 1) // block
    out = torch.empty((B, Hkv, L, d), dtype=dtype)
    scale = torch.empty((B, Hkv, nblk), dtype=F32)
    pad = nblk * block - L
    for b in range(B):
        for h in range(Hkv):
            slab = torch.randn((L, d), generator=g, dtype=F32)
            amp = torch.exp2(torch.rand((nblk,), generator=g, dtype=F32) * 4 - 2)
            slab.mul_(amp.repeat_interleave(block)[:L, None])
            amax = torch.nn.functional.pad(slab.abs(), (0, 0, 0, pad)).view(nblk, block * d).amax(dim=1)
            scale[b, h] = (amax.double() / FP8_MAX[dtype]).float()
            out[b, h].copy_((slab / scale[b, h].repeat_interleave(block)[:L, None]).to(dtype))
    return out, scale


def draw_seq_lens(seed: int, B: int, lo: int, hi: int) -> torch.Tensor:
    """Integers uniform on [lo, hi] inclusive, int32."""
    return torch.randint(lo, hi + 1, (B,), generator=_gen(seed), dtype=torch.int64).to(torch.int32)


def make_workload(wid: int, scale_block: int = 0):
    """All inputs of workload ``wid`` as CPU tensors.

    Returns a dict with q, k, v, seq_lens (int32 or None), slopes (fp32 or None),
    n_splits (int, <= 0 for automatic) and, for workload 5, planted (int64 [B, Hkv]).
    ``scale_block`` > 0 (FP8 workloads): K and V quantised per block of that many keys
    by ``draw_kv_fp8_blocks`` (same seeds), scales [B, Hkv, ceil(Lmax / scale_block)].
    """
    w = WORKLOADS[wid]
    base = 1000 * wid
    q = draw_q(base + 0, w.B, w.Hq, w.d, w.q_dtype)
    ks = vs = None
    if w.kv_dtype in FP8_MAX and scale_block > 0:
        k, ks = draw_kv_fp8_blocks(base + 1, w.B, w.Hkv, w.Lmax, w.d, scale_block, w.kv_dtype)
        v, vs = draw_kv_fp8_blocks(base + 2, w.B, w.Hkv, w.Lmax, w.d, scale_block, w.kv_dtype)
    elif w.kv_dtype in FP8_MAX:
        k, ks = draw_kv_fp8(base + 1, w.B, w.Hkv, w.Lmax, w.d, w.kv_dtype)
        v, vs = draw_kv_fp8(base + 2, w.B, w.Hkv, w.Lmax, w.d, w.kv_dtype)
    else:
        k = draw_kv(base + 1, w.B, w.Hkv, w.Lmax, w.d, w.kv_dtype, w.k_scale)
        v = draw_kv(base + 2, w.B, w.Hkv, w.Lmax, w.d, w.kv_dtype)
    seq_lens = None
    if w.ragged:
        seq_lens = draw_seq_lens(base + 3, w.B, w.ragged_lo, w.Lmax)
        for b in range(w.B):
            L = int(seq_lens[b])
            if w.kv_dtype in FP8_MAX:                 # the format's NaN bit pattern
                k.view(torch.uint8)[b, :, L:, :] = _nan_bits(w.kv_dtype)
                v.view(torch.uint8)[b, :, L:, :] = _nan_bits(w.kv_dtype)
            else:
                k[b, :, L:, :] = float("nan")
                v[b, :, L:, :] = float("nan")
    slopes = alibi_slopes(w.Hq) if w.alibi else None
    planted = None
    if w.planted_logit is not None:
        planted = plant_dominant_keys(base + 4, q, k, w.planted_logit)
    return dict(workload=w, q=q, k=k, v=v, seq_lens=seq_lens, slopes=slopes,
                n_splits=w.n_splits, planted=planted, k_scale=ks, v_scale=vs)


def plant_dominant_keys(seed: int, q: torch.Tensor, k: torch.Tensor, logit: float) -> torch.Tensor:
    """Replace one key per (b, kv-head) at a seeded position by bf16(c * q_h).

    The query head used is the first of the KV head's group; c = logit*sqrt(d)/|q_h|^2,
    so the planted key's scaled score is close to ``logit``.  Returns positions [B, Hkv].
    """
    B, Hkv, L, d = k.shape
    g = _gen(seed)
    pos = torch.randint(0, L, (B, Hkv), generator=g, dtype=torch.int64)
    group = q.shape[1] // Hkv
    for b in range(B):
        for h in range(Hkv):
            qh = q[b, h * group].to(torch.float64)
            c = logit * math.sqrt(d) / float((qh * qh).sum())
            k[b, h, int(pos[b, h])] = (c * qh).to(k.dtype)
    return pos


def random_case(seed: int, B: int, Hq: int, Hkv: int, L: int, d: int, q_dtype=F32, kv_dtype=BF16,
                seq_lens=None, alibi: bool = False, k_scale: float = 1.0, poison_tail: bool = True,
                scale_block: int = 0):
    """A small seeded case of arbitrary shape for parity tests (same recipe as the workloads).

    FP8 K/V (kv_dtype float8_e4m3fn / float8_e5m2) come with per-(b, kv-head) scales in
    the returned k_scale / v_scale (None otherwise), or, with ``scale_block`` > 0, with
    per-(b, kv-head, key block) scales [B, Hkv, ceil(L / scale_block)] from
    ``draw_kv_fp8_blocks``."""
    q = draw_q(seed, B, Hq, d, q_dtype)
    ks = vs = None
    if kv_dtype in FP8_MAX and scale_block > 0:
        k, ks = draw_kv_fp8_blocks(seed + 1, B, Hkv, L, d, scale_block, kv_dtype)
        v, vs = draw_kv_fp8_blocks(seed + 2, B, Hkv, L, d, scale_block, kv_dtype)
        if k_scale != 1.0:
            ks = ks * k_scale
    elif kv_dtype in FP8_MAX:
        k, ks = draw_kv_fp8(seed + 1, B, Hkv, L, d, kv_dtype)
        v, vs = draw_kv_fp8(seed + 2, B, Hkv, L, d, kv_dtype)
        if k_scale != 1.0:
            ks = ks * k_scale
    else:
        k = draw_kv(seed + 1, B, Hkv, L, d, kv_dtype, k_scale)
        v = draw_kv(seed + 2, B, Hkv, L, d, kv_dtype)
    sl = None
    if seq_lens is not None:
        sl = torch.as_tensor(seq_lens, dtype=torch.int32)
        if poison_tail:
            for b in range(B):
                Lb = max(0, min(int(sl[b]), L))
                if kv_dtype in FP8_MAX:       # NaN bit patterns (E4M3: 0x7F, E5M2: 0x7E)
                    nan_bits = 0x7F if kv_dtype == torch.float8_e4m3fn else 0x7E
                    k.view(torch.uint8)[b, :, Lb:, :] = nan_bits
                    v.view(torch.uint8)[b, :, Lb:, :] = nan_bits
                else:
                    k[b, :, Lb:, :] = float("nan")
                    v[b, :, Lb:, :] = float("nan")
    slopes = alibi_slopes(Hq) if alibi else None
    return dict(q=q, k=k, v=v, seq_lens=sl, slopes=slopes, k_scale=ks, v_scale=vs)


def _raw(t: torch.Tensor) -> torch.Tensor:
    """Bit view (int16 for 2-byte, uint8 for 1-byte, int32 for 4-byte elements)."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def _nan_bits(dtype) -> int:
    if dtype == torch.float8_e4m3fn:
        return 0x7F
    if dtype == torch.float8_e5m2:
        return 0x7E
    return int(torch.tensor(float("nan"), dtype=dtype).view({2: torch.int16, 4: torch.int32}[
        torch.tensor(0, dtype=dtype).element_size()]))


def page_kv(k: torch.Tensor, v: torch.Tensor, page_size: int, seed: int, spare: int = 3,
            head_major: bool = False):
    """Copy [B, Hkv, L, d] K and V into a paged cache.

    Returns (k_cache, v_cache, block_table): caches shaped [num_pages, page_size, Hkv, d]
    with num_pages = B * ceil(L / page_size) + spare, and block_table int32
    [B, ceil(L / page_size)] whose entry [b, p] is the page holding logical rows
    [p * page_size, (p + 1) * page_size) of batch row b.  Pages are handed out by a
    seeded random permutation of the pool; rows no logical key maps to (spare pages,
    the tail of the last page) hold NaN.  head_major stores each page as
    [Hkv, page_size, d] (the returned caches are then strided views of that storage).
    Pure data movement, on bit views: values are copied exactly."""
    B, Hkv, L, d = k.shape
    mp = max(1, -(-L // page_size))
    n_pages = B * mp + spare
    perm = torch.randperm(n_pages, generator=_gen(seed + 5))
    table = perm[:B * mp].view(B, mp).to(torch.int32)
    caches = []
    for x in (k, v):
        fill = _nan_bits(x.dtype)
        padded = torch.full((B, Hkv, mp * page_size, d), fill, dtype=_raw(x).dtype)
        padded[:, :, :L] = _raw(x)
        pages = padded.view(B, Hkv, mp, page_size, d)
        if head_major:
            store = torch.full((n_pages, Hkv, page_size, d), fill, dtype=padded.dtype)
            store[table.view(-1).long()] = pages.permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, page_size, d)
            cache = store.view(x.dtype).permute(0, 2, 1, 3)
        else:
            store = torch.full((n_pages, page_size, Hkv, d), fill, dtype=padded.dtype)
            store[table.view(-1).long()] = pages.permute(0, 2, 3, 1, 4).reshape(B * mp, page_size, Hkv, d)
            cache = store.view(x.dtype)
        caches.append(cache)
    return caches[0], caches[1], table
