// split_valu.hip -- split step of split-KV decoding on the vector ALUs (gfx950).
//
// One work-group (4 waves) owns one (batch row b, query head h, chunk s).  The chunk
// is the s-th of the row's L_b keys cut into pieces of one batch-wide length (see
// chunk_range in tad_internal.h; torch.chunk(S) for a single length).  It produces the chunk's
// partial (m, l, o): the local maximum of the scores, the sum of exponentials
// relative to it, and the exponential-weighted sum of value rows -- the
// (local_max, den, num) triple of tree_attn_decode in "Tree Attention Decoding",
// with the maximum and the exponentials in base 2 (the query is pre-scaled by
// d^-1/2 * log2 e so that exp(x) becomes 2^x on the transcendental unit).
//
// Inside the chunk the keys stream through registers in tiles; each tile updates a
// running maximum and sum in the manner of the block loop in "Flash Aandacht"
// (section "Implementatiedetails"), but the output accumulator is kept
// un-normalised -- rescaled by 2^(m_old - m_new) only -- and divided once, in the
// merge step.  (The page's listing divides by the new running sum every block
// without first multiplying the old output back by the old sum, which is only right
// when the whole sequence fits in one block.)
//
// Lane layout: a key row of d elements is spread over G = d/EPL lanes, each holding
// EPL consecutive elements (8 for fp32 and bf16, 16 for FP8: one 16-byte load, two
// for fp32).  A wave therefore covers 64/G keys per load instruction; the q.k dot
// product is EPL FMAs per lane followed by a log2(G)-step DPP butterfly inside the
// lane group.  FP8 K/V carry a dequantisation scale per (b, kv head) -- the K scale
// folded into q, the V scale into the chunk's output -- or per block of key positions:
// then a load's KPW keys share one block (blocks hold at least 16 keys and chunks and
// pieces start on block boundaries), whose K scale multiplies their scores and whose
// V scale their value weights, one scalar load each per tile and load.  Each lane group
// runs its own online softmax over the keys it sees (no cross-group traffic in the
// loop); the 4*64/G group states of a work-group are merged through LDS at the end.
//
// HBM traffic: every K and V byte of the chunk is read exactly once with 16-byte
// coalesced buffer loads; loads past the chunk end return zero (buffer range), so
// ragged tails and neighbouring chunks are never fetched.

#include "device_util.h"
#include "merge.h"
#include "tad_internal.h"

namespace tad {

// POLICY: kPolicyNT when every K/V byte is read by one work-group only (one query
// head per KV head); the default policy when the g work-groups of a query-head group
// re-read the same chunk and should find it in L2.
// UK: keys per lane group per tile (K and V tiles of UK*16 bytes per lane for bf16).
// KVT: element type of K and V (kKvF32, kKvBF16, kKvE4M3, kKvE5M2).
// PAGED: K/V rows come from a paged cache through the block table; a wave tile is one
// or two pieces of 16 rows, each inside one page (page sizes are multiples of 16) with
// its own buffer resource.
// TAIL: the variant whose last work-group of a row also merges the row (a.fused), kept
// apart so that the plain kernel carries none of that code or its registers.
// BLK: FP8 K/V with block scales (likewise kernels of their own).
template <int D, int KVT, int POLICY, int UK = 128 / RowChunk<KVT, POLICY>::kBytes, bool PAGED = false,
          bool TAIL = false, bool BLK = false>
__global__ __launch_bounds__(kSplitThreads) void split_valu_kernel(SplitArgs a) {
    using Row = RowChunk<KVT, POLICY>;
    constexpr bool F8 = KVT == kKvE4M3 || KVT == kKvE5M2;
    static_assert(!BLK || F8, "block scales are for FP8 K/V");
    constexpr int EPL = Row::EPL;                // elements per lane per key
    constexpr int G = D / EPL;                   // lanes per key row
    constexpr int KPW = 64 / G;                  // keys per wave load instruction
    constexpr int ELEM = KVT == kKvF32 ? 4 : (KVT == kKvBF16 ? 2 : 1);
    constexpr int U = UK;                        // keys per lane group per tile
    constexpr int T = KPW * U;                   // keys per wave tile
    constexpr int NW = kSplitThreads / 64;       // waves per work-group
    constexpr int SLOTS = NW * KPW;              // lane-group states to merge
    // paged: a tile is 1 or 2 pieces of 16 rows, each inside one page (page sizes are
    // multiples of 16), each with its own block-table lookup
    constexpr int NSUB = PAGED ? T / 16 : 1;
    static_assert(!PAGED || ((T == 16 || T == 32) && 16 % KPW == 0), "paged tiles: 16-row pieces");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int grp = lane / G;
    const int sub = lane % G;

    // ---- work-group -> (b, h, t, s, p): query head h, query token t, chunk s, piece p
    // of the chunk (pieces: one query row per KV head only).  When several (head,
    // token) rows read the same KV chunk (query-head groups, several tokens), their gq
    // work-groups get ids that are equal modulo 8, so they land on the same XCD and
    // share its L2.
    int b, h, t, s, p = 0;
    const int S = a.S;
    const int gq = a.group * a.nq;                        // rows per KV head
    if (gq == 1) {
        int id = blockIdx.x;
        p = id % a.P;
        id /= a.P;
        s = id % S;
        const int row = id / S;
        b = row / a.Hq;
        h = row % a.Hq;
        t = 0;
    } else {
        const int id = blockIdx.x;
        const int xcd = id & 7;
        const int slot = id >> 3;
        const int r = slot % gq;
        const int u = (slot / gq) * 8 + xcd;              // (b, kvh, s) unit
        if (u >= a.B * a.Hkv * S) return;
        s = u % S;
        const int bk = u / S;
        b = bk / a.Hkv;
        h = (bk % a.Hkv) * a.group + r / a.nq;
        t = r % a.nq;
    }
    const int kvh = h / a.group;

    // The chunk (or its piece p) of the KV row, clipped to the keys this token sees;
    // from here on the row is single-token decode over its first L keys.
    const int cfull = batch_chunk_len(a);
    ChunkRange cr = chunk_of(row_len(a, b), s, cfull);
    if (a.P > 1) {
        const int cs = sub_chunk_len(a, cfull);
        const int pj0 = (int)min((int64_t)cr.j0 + (int64_t)p * cs, (int64_t)cr.j1);
        cr.j1 = min(pj0 + cs, cr.j1);
        cr.j0 = pj0;
    }
    const int L = visible_keys(cr.L, a.nq, t);
    const int j1 = min(cr.j1, L), j0 = min(cr.j0, j1);
    const int n = j1 - j0;

    // ---- buffer resources: one per chunk ([chunk start, chunk end) of this head's K
    // and V), or, for a paged cache, one per tile (built in load_tile).
    const KvRows kvk(a.k, ELEM, a.skb, a.skh, a.skj, a.skp, a, b, kvh);
    const KvRows kvv(a.v, ELEM, a.svb, a.svh, a.svj, a.svp, a, b, kvh);
    const uint32_t krow = kvk.row_bytes, vrow = kvv.row_bytes;
    const __amdgpu_buffer_rsrc_t kr = PAGED ? make_rsrc(nullptr, 0u) : kvk.rows(j0, n);
    const __amdgpu_buffer_rsrc_t vr = PAGED ? make_rsrc(nullptr, 0u) : kvv.rows(j0, n);
    TilePages pages[NSUB];                                 // paged: this wave's tile pages

    // ---- this lane's EPL query elements, pre-scaled into base-2 units (and by the
    // K dequantisation scale, which multiplies every score of this KV head).
    float qv[EPL];
    {
        const bool k_head = a.k_scale && (!BLK || !a.k_blk_lg);   // one K scale per (b, KV head)
        const float qs = a.qscale * (k_head ? a.k_scale[b * a.Hkv + kvh] : 1.f);
        const int64_t qoff = (int64_t)b * a.sqb + (int64_t)h * a.sqh + (int64_t)t * a.sqt + sub * EPL;
#pragma unroll
        for (int c8 = 0; c8 < EPL / 8; ++c8) {
            if (a.q_bf16) {
                const uint4 w = *(const uint4 *)((const uint16_t *)a.q + qoff + 8 * c8);
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qv[8 * c8 + 2 * i] = bf16_lo(ws[i]) * qs;
                    qv[8 * c8 + 2 * i + 1] = bf16_hi(ws[i]) * qs;
                }
            } else {
                const float4 *qp = (const float4 *)((const float *)a.q + qoff + 8 * c8);
                const float4 x0 = qp[0], x1 = qp[1];
                qv[8 * c8 + 0] = x0.x * qs; qv[8 * c8 + 1] = x0.y * qs;
                qv[8 * c8 + 2] = x0.z * qs; qv[8 * c8 + 3] = x0.w * qs;
                qv[8 * c8 + 4] = x1.x * qs; qv[8 * c8 + 5] = x1.y * qs;
                qv[8 * c8 + 6] = x1.z * qs; qv[8 * c8 + 7] = x1.w * qs;
            }
        }
    }
    // ALiBi in base-2 units: bias of key j is slope*log2e*(j - (L-1)); j - (L-1) is an
    // exact integer in fp32 for L < 2^24.
    const float slope2 = a.slopes ? a.slopes[h] * 1.4426950408889634f : 0.f;
    const bool alibi = a.slopes != nullptr;

    float m = kNegInf, l = 0.f;
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    const uint32_t lane_off = (uint32_t)(sub * EPL * ELEM);
    using Tile = Row[U];
    auto load_tile = [&](Tile &kk, Tile &vv, int t0) {
        if constexpr (PAGED) {
            // piece h: rows [16 h, 16 h + 16) of the tile, from its own page
            __amdgpu_buffer_rsrc_t krs[NSUB], vrs[NSUB];
            const int k = (t0 - wave * T) / (NW * T);      // this wave's tile number
#pragma unroll
            for (int h = 0; h < NSUB; ++h) {
                const int th = t0 + 16 * h;
                const int nt = max(0, min(16, n - th));
                const int page = pages[h].get(kvk, j0, n, wave * T + 16 * h, NW * T, k);
                krs[h] = kvk.page_rows(page, j0 + th, nt);
                vrs[h] = kvv.page_rows(page, j0 + th, nt);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                constexpr int RPP = 16 / KPW;               // load instructions per piece
                const int h = u / RPP, r = (u % RPP) * KPW + grp;
                kk[u].load(krs[h], (uint32_t)r * krow + lane_off);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                constexpr int RPP = 16 / KPW;
                const int h = u / RPP, r = (u % RPP) * KPW + grp;
                vv[u].load(vrs[h], (uint32_t)r * vrow + lane_off);
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) kk[u].load(kr, (uint32_t)(t0 + u * KPW + grp) * krow + lane_off);
#pragma unroll
            for (int u = 0; u < U; ++u) vv[u].load(vr, (uint32_t)(t0 + u * KPW + grp) * vrow + lane_off);
        }
    };
    // One tile: scores, online max/sum update, value accumulation.
    auto consume = [&](const Tile &kk, const Tile &vv, int t0) {
        float sc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[EPL];
            kk[u].widen(kf);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc = fmaf(qv[e], kf[e], acc);
            sc[u] = group_sum<G>(acc);
        }
        float vsu[U];                                       // V block scales of the tile's loads
        if constexpr (BLK) {
            const int bkv = b * a.Hkv + kvh;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ju = __builtin_amdgcn_readfirstlane(j0 + t0 + u * KPW);
                if (a.k_blk_lg) sc[u] *= block_scale(a.k_scale, a.k_blk_lg, a.k_nblk, bkv, ju);
                vsu[u] = a.v_blk_lg ? block_scale(a.v_scale, a.v_blk_lg, a.v_nblk, bkv, ju) : 1.f;
            }
        }
        if (alibi) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                sc[u] = fmaf(slope2, (float)(j0 + t0 + u * KPW + grp - (L - 1)), sc[u]);
        }
        if (t0 + T > n) {                                   // tail tile: mask keys past the chunk
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (t0 + u * KPW + grp >= n) sc[u] = kNegInf;
        }
        float mt = sc[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mt = fmaxf(mt, sc[u]);
        const float m_new = fmaxf(m, mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;   // all masked so far: no NaN
        const float alpha = exp2_fast(m - m_use);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = exp2_fast(sc[u] - m_use);
            l += p;
            float pv = p;
            if constexpr (BLK) pv = p * vsu[u];
            float vf[EPL];
            vv[u].widen(vf);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = fmaf(pv, vf[e], o[e]);
        }
        m = m_new;
    };

    constexpr int STRIDE = NW * T;
    for (int t0 = wave * T; t0 < n; t0 += STRIDE) {
        Tile kk, vv;
        load_tile(kk, vv, t0);
        consume(kk, vv, t0);
    }

    // ---- merge the SLOTS lane-group states of this work-group (fixed order).
    __shared__ float lds_o[SLOTS][D];
    __shared__ float lds_m[SLOTS], lds_l[SLOTS];
    const int slot = wave * KPW + grp;
#pragma unroll
    for (int e = 0; e < EPL; ++e) lds_o[slot][sub * EPL + e] = o[e];
    if (sub == 0) {
        lds_m[slot] = m;
        lds_l[slot] = l;
    }
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) M = fmaxf(M, lds_m[i]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    const int64_t row = ((int64_t)b * a.Hq + h) * a.nq + t;
    const int64_t r = row * S + s;
    const bool v_head = a.v_scale && (!BLK || !a.v_blk_lg);
    const float vsc = v_head ? a.v_scale[b * a.Hkv + kvh] : 1.f;   // V dequantisation
    // Where this work-group's partial goes: the chunk's slot, or piece p's slot (a later
    // kernel merges the pieces).  A partial that another work-group of this kernel
    // merges (fused) is written through to the device coherence point (store_partial).
    const bool piece = a.P > 1;
    const int64_t rp = r * a.P + p;
    float *const pm = piece ? a.sub_m + rp : a.ws_m + r;
    float *const pl = piece ? a.sub_l + rp : a.ws_l + r;
    float *const po = piece ? a.sub_o + rp * D : a.ws_o + r * D;
    for (int e = threadIdx.x; e < D; e += kSplitThreads) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) acc = fmaf(exp2_fast(lds_m[i] - Mu), lds_o[i][e], acc);
        acc *= vsc;
        if constexpr (TAIL) store_partial(po + e, acc);
        else po[e] = acc;
    }
    if (threadIdx.x == 0) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) acc = fmaf(exp2_fast(lds_m[i] - Mu), lds_l[i], acc);
        if constexpr (TAIL) {
            store_partial(pm, M);
            store_partial(pl, acc);
        } else {
            *pm = M;
            *pl = acc;
        }
    }

    if constexpr (TAIL) {
        static_assert(SLOTS * D >= kMaxFusedSplits + kMergeThreads, "merge scratch fits in lds_o");
        __shared__ int last;
        // ---- fused merge: the last of the row's S work-groups to finish merges the row.
        if (arrive_last(&a.cnt[row], S, &last)) {
            merge_row<D, true>(a.ws_m + row * S, a.ws_l + row * S, a.ws_o + row * S * D, S,
                               a.out + (int64_t)b * a.sob + (int64_t)h * a.soh + (int64_t)t * a.sot,
                               &lds_o[0][0]);
            reset_counter(&a.cnt[row]);
        }
    }
}

template <int D, int KVT, bool TAIL, bool BLK>
static hipError_t launch_tail(const SplitArgs &a, int64_t grid, hipStream_t st) {
    // paged caches: 32-key wave tiles of two 16-row pieces, each from its own page (page
    // sizes are multiples of 16), or 16 keys where 32 would take more than 8 loads per
    // lane and tensor (4 for FP8, as on contiguous caches).  32 heads x 131072 bf16 keys
    // in head-major pages, per step: 16-row pages 335.7-336.4 -> 330.2-332.4 us, 64-row
    // pages 332.5-334.9 -> 324.3-324.8 us against 16-key tiles.
    constexpr int KPW = 64 * RowChunk<KVT, kPolicyNT>::EPL / D;
    constexpr bool F8 = KVT == kKvE4M3 || KVT == kKvE5M2;
    constexpr int UP = 32 / KPW <= (F8 ? 4 : 8) ? 32 / KPW : 16 / KPW;
    // contiguous caches: 128 bytes of each row per lane and tensor in flight (8 loads),
    // except FP8, whose rows take twice the arithmetic per byte: 4 loads (one row of 32
    // heads x 131072 keys of E4M3: 164.0-164.4 us per step against 168.0-168.2 us with
    // 8, 170-171 with 2, 172-173 with 3)
    constexpr int UD = F8 ? 4 : 128 / RowChunk<KVT, kPolicyNT>::kBytes;
    const int gq = a.group * a.nq;
    if (a.block_table) {
        if constexpr (KVT == kKvF32 || D > 256) {
            return hipErrorInvalidValue;                  // not offered for paged caches
        } else if (gq == 1) {
            hipLaunchKernelGGL((split_valu_kernel<D, KVT, kPolicyNT, UP, true, TAIL, BLK>), dim3((unsigned)grid),
                               dim3(kSplitThreads), 0, st, a);
        } else {
            hipLaunchKernelGGL((split_valu_kernel<D, KVT, kPolicyDefault, UP, true, TAIL, BLK>),
                               dim3((unsigned)grid), dim3(kSplitThreads), 0, st, a);
        }
    } else if (gq == 1) {
        hipLaunchKernelGGL((split_valu_kernel<D, KVT, kPolicyNT, UD, false, TAIL, BLK>), dim3((unsigned)grid),
                           dim3(kSplitThreads), 0, st, a);
    } else {
        hipLaunchKernelGGL((split_valu_kernel<D, KVT, kPolicyDefault, UD, false, TAIL, BLK>), dim3((unsigned)grid),
                           dim3(kSplitThreads), 0, st, a);
    }
    return hipGetLastError();
}

template <int D, int KVT, bool BLK = false>
static hipError_t launch_t(const SplitArgs &a, hipStream_t st) {
    int64_t grid;
    const int gq = a.group * a.nq;
    if (a.P > 1 && gq != 1) return hipErrorInvalidValue;   // pieces: one query row per KV head only
    if (gq == 1) {
        grid = (int64_t)a.B * a.Hq * a.S * a.P;
    } else {
        const int64_t units = (int64_t)a.B * a.Hkv * a.S;
        grid = (units + 7) / 8 * 8 * gq;
    }
    if (grid <= 0) return hipSuccess;
    if (a.fused && a.P > 1) return hipErrorInvalidValue;   // pieces merge in their own kernel
    if (a.fused) return launch_tail<D, KVT, true, BLK>(a, grid, st);
    return launch_tail<D, KVT, false, BLK>(a, grid, st);
}

template <int D>
static hipError_t launch_d(const SplitArgs &a, hipStream_t st) {
    const bool blk = a.k_blk_lg || a.v_blk_lg;         // FP8 block scales: kernels of their own
    switch (a.kv_type) {
        case kKvF32: return launch_t<D, kKvF32>(a, st);
        case kKvBF16: return launch_t<D, kKvBF16>(a, st);
        case kKvE4M3: return blk ? launch_t<D, kKvE4M3, true>(a, st) : launch_t<D, kKvE4M3>(a, st);
        case kKvE5M2: return blk ? launch_t<D, kKvE5M2, true>(a, st) : launch_t<D, kKvE5M2>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_split_valu(const SplitArgs &a, int d, hipStream_t st) {
    switch (d) {
        case 64: return launch_d<64>(a, st);
        case 128: return launch_d<128>(a, st);
        case 256: return launch_d<256>(a, st);
        case 512: return launch_d<512>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tad
