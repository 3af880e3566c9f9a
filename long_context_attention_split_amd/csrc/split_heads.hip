// split_heads.hip -- split step for K/V caches whose heads are interleaved per token.
//
// Same chunk partials (m, l, o) as split_valu.hip -- the per-chunk (local max,
// denominator, numerator) of tree_attn_decode in "Tree Attention Decoding", maximum
// and exponentials in base 2 -- for one query head per KV head and one query token,
// when the cache stores the heads of a token next to each other ([B, L, Hkv, d] seen
// through strides, or pages of [page_size, Hkv, d]).  There a (head, key) row is a
// short run (256 bytes for bf16, d = 128) at a stride of Hkv rows, and a kernel that
// reads one head at a time issues short, widely spaced runs that HBM serves well
// below its streaming rate.
//
// Here a wave's load instruction covers 4 adjacent heads of one key instead: a head
// row is spread over 16 lanes (d/16 elements each), and the wave reads 4 d
// contiguous elements per key (1 KiB for bf16 at d = 128).  Each 16-lane group runs
// the online softmax of its own head over the keys of its wave's tiles; the 16 waves
// of a work-group take interleaved tiles of the same chunk and merge their states
// per head through LDS at the end.  A launch (B * Hq / 4 * S work-groups of 16 waves)
// has as many waves as split_valu's for the same chunk count.
//
// FP8 block scales: a tile's U keys (a power of two, at most 16) lie in one block, since
// blocks hold at least 16 keys and chunks start on block boundaries, so each lane group
// loads its head's K and V scale once per tile, one tile ahead.
//
// Every K and V byte of a chunk is read once, with 16-byte buffer loads; loads past
// the chunk end return zero.  Every chunk has its work-group, so an empty chunk writes
// the merge identity (m = -inf, l = 0, o = 0) itself.

#include "device_util.h"
#include "merge.h"
#include "tad_internal.h"

namespace tad {

// One lane's slice of one (head, key) row: EPL = d / 16 consecutive elements (a head
// row is spread over 16 lanes), BYTES = EPL * element size in {4, 8, 16, 32, 64},
// loaded with one 4- or 8-byte load or 16-byte loads, widened to fp32.
template <int KVT, int EPL>
struct HeadSlice {
    static constexpr int ELEM = KVT == kKvF32 ? 4 : (KVT == kKvBF16 ? 2 : 1);
    static constexpr int BYTES = EPL * ELEM;
    static constexpr int WORDS = BYTES / 4;
    uint32_t w[WORDS];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        if constexpr (BYTES == 4) {
            w[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicyNT);
        } else if constexpr (BYTES == 8) {
            typedef unsigned u2_t __attribute__((ext_vector_type(2)));
            const u2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicyNT);
            w[0] = x.x;
            w[1] = x.y;
        } else {
#pragma unroll
            for (int i = 0; i < BYTES / 16; ++i) {
                const uint4 x = load16<kPolicyNT>(r, off + 16u * i);
                w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
            }
        }
    }
    __device__ __forceinline__ void widen(float (&f)[EPL]) const {
        if constexpr (KVT == kKvF32) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) f[i] = __uint_as_float(w[i]);
        } else if constexpr (KVT == kKvBF16) {
#pragma unroll
            for (int i = 0; i < WORDS; ++i) {
                f[2 * i] = bf16_lo(w[i]);
                f[2 * i + 1] = bf16_hi(w[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < WORDS; ++i) {
                typedef float f2_t __attribute__((ext_vector_type(2)));
                f2_t lo, hi;
                if constexpr (KVT == kKvE4M3) {
                    lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
                    hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
                } else {
                    lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w[i], false);
                    hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w[i], true);
                }
                f[4 * i] = lo.x; f[4 * i + 1] = lo.y; f[4 * i + 2] = hi.x; f[4 * i + 3] = hi.y;
            }
        }
    }
};

constexpr int kHeadLanes = 16;                   // lanes per head row
constexpr int kHeadsPerWave = 64 / kHeadLanes;   // 4
constexpr int kHeadsWaves = 16;                  // waves per work-group
constexpr int kHeadsThreads = 64 * kHeadsWaves;

// TAIL: the one-launch form (a.fused).  The work-groups write their partials through to
// the device coherence point, and the last of a (b, 4-head group)'s S chunks to arrive
// (arrive_last: agent-scope acq_rel ticket on the group's counter) merges the group's 4
// rows with merge_rows -- the combine's arithmetic, so the same bits -- and returns
// the counter to zero.
// BLK: FP8 K/V with block scales (kernels of their own, so that the per-(b, KV head)
// kernels keep their registers and schedule).
template <int D, int KVT, bool PAGED, bool TAIL = false, bool BLK = false>
__global__ __launch_bounds__(kHeadsThreads) void split_heads_kernel(SplitArgs a) {
    constexpr int G = kHeadLanes, HPW = kHeadsPerWave, NW = kHeadsWaves;
    constexpr int EPL = D / G;
    using Row = HeadSlice<KVT, EPL>;
    constexpr bool F8 = KVT == kKvE4M3 || KVT == kKvE5M2;
    static_assert(!BLK || F8, "block scales are for FP8 K/V");
    // keys per wave tile (a power of two <= 16, so it divides every page size): K and
    // V tiles of 16 KiB per wave for bf16 slices up to 16 bytes, 8 KiB otherwise --
    // FP8 widening and 16-element slices need the registers
    constexpr int TILE_BYTES = (KVT == kKvBF16 && Row::BYTES <= 16) ? 128 : 64;
    constexpr int U = TILE_BYTES / Row::BYTES < 16 ? TILE_BYTES / Row::BYTES : 16;
    constexpr int STRIDE = NW * U;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int grp = lane / G;                    // head h0 + grp
    const int sub = lane % G;

    // ---- work-group -> (b, heads [h0, h0 + HPW), chunk s)
    const int S = a.S;
    const int s = blockIdx.x % S;
    const int bh = blockIdx.x / S;
    const int n_hb = a.Hq / HPW;
    const int b = bh / n_hb;
    const int h0 = (bh % n_hb) * HPW;
    const int h = h0 + grp;                      // query head = KV head (group 1)

    const ChunkRange cr = chunk_range(a, b, s);
    const int j0 = cr.j0, n = cr.j1 - cr.j0;
    const int L = cr.L;

    // Resources start at head h0 of the chunk's first key: a key's HPW heads are the
    // HPW * D contiguous elements from there.
    const KvRows kvk(a.k, Row::ELEM, a.skb, a.skh, a.skj, a.skp, a, b, h0);
    const KvRows kvv(a.v, Row::ELEM, a.svb, a.svh, a.svj, a.svp, a, b, h0);
    const uint32_t krow = kvk.row_bytes, vrow = kvv.row_bytes;
    const __amdgpu_buffer_rsrc_t kr = PAGED ? make_rsrc(nullptr, 0u) : kvk.rows(j0, n);
    const __amdgpu_buffer_rsrc_t vr = PAGED ? make_rsrc(nullptr, 0u) : kvv.rows(j0, n);

    // ---- this lane's EPL query elements of head h, in base-2 units, times the K
    // dequantisation scale of the head.
    float qv[EPL];
    {
        const bool k_head = a.k_scale && (!BLK || !a.k_blk_lg);   // one K scale per (b, KV head)
        const float qs = a.qscale * (k_head ? a.k_scale[b * a.Hkv + h] : 1.f);
        const int64_t qoff = (int64_t)b * a.sqb + (int64_t)h * a.sqh + sub * EPL;
        if (a.q_bf16) {
            const uint16_t *qp = (const uint16_t *)a.q + qoff;
#pragma unroll
            for (int e = 0; e < EPL; ++e) qv[e] = __uint_as_float((uint32_t)qp[e] << 16) * qs;
        } else {
            const float *qp = (const float *)a.q + qoff;
#pragma unroll
            for (int e = 0; e < EPL; ++e) qv[e] = qp[e] * qs;
        }
    }
    const float slope2 = a.slopes ? a.slopes[h] * 1.4426950408889634f : 0.f;
    const bool alibi = a.slopes != nullptr;

    float m = kNegInf, l = 0.f;
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    const uint32_t lane_off = (uint32_t)(lane * Row::BYTES);
    TilePages pages;                                       // paged: this wave's tile pages
    // BLK: the block scales of the tile at t (its U keys lie in one block), for this
    // lane group's head; each tile's are loaded one tile ahead, behind the K and V rows
    // of the tile before.
    float kst = 1.f, vst = 1.f;
    auto tile_scales = [&](int t, float &ks, float &vs) {
        const int jt = __builtin_amdgcn_readfirstlane(j0 + t);
        if (a.k_blk_lg) ks = block_scale(a.k_scale, a.k_blk_lg, a.k_nblk, b * a.Hkv + h, jt);
        if (a.v_blk_lg) vs = block_scale(a.v_scale, a.v_blk_lg, a.v_nblk, b * a.Hkv + h, jt);
    };
    if constexpr (BLK) tile_scales(wave * U, kst, vst);
    for (int t0 = wave * U, k = 0; t0 < n; t0 += STRIDE, ++k) {
        __amdgpu_buffer_rsrc_t krs = kr, vrs = vr;
        int tb = t0;                                       // first key, relative to the resource
        if constexpr (PAGED) {
            const int nt = min(U, n - t0);                 // the tile lies in one page
            const int page = pages.get(kvk, j0, n, wave * U, STRIDE, k);
            krs = kvk.page_rows(page, j0 + t0, nt);
            vrs = kvv.page_rows(page, j0 + t0, nt);
            tb = 0;
        }
        Row kk[U], vv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) kk[u].load(krs, (uint32_t)(tb + u) * krow + lane_off);
#pragma unroll
        for (int u = 0; u < U; ++u) vv[u].load(vrs, (uint32_t)(tb + u) * vrow + lane_off);
        float kstn = 1.f, vstn = 1.f;                      // BLK: the next tile's scales
        if constexpr (BLK) tile_scales(t0 + STRIDE, kstn, vstn);

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
        if constexpr (BLK) {
#pragma unroll
            for (int u = 0; u < U; ++u) sc[u] *= kst;
        }
        if (alibi) {
#pragma unroll
            for (int u = 0; u < U; ++u) sc[u] = fmaf(slope2, (float)(j0 + t0 + u - (L - 1)), sc[u]);
        }
        if (t0 + U > n) {                                  // tail tile: mask keys past the chunk
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (t0 + u >= n) sc[u] = kNegInf;
        }
        float mt = sc[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mt = fmaxf(mt, sc[u]);
        const float m_new = fmaxf(m, mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2_fast(m - m_use);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = exp2_fast(sc[u] - m_use);
            l += p;
            float pv = p;
            if constexpr (BLK) pv = p * vst;
            float vf[EPL];
            vv[u].widen(vf);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = fmaf(pv, vf[e], o[e]);
        }
        m = m_new;
        if constexpr (BLK) {
            kst = kstn;
            vst = vstn;
        }
    }

    // ---- merge the NW wave states of each head (fixed order) and write the partials.
    __shared__ __align__(16) float lds_o[NW][HPW * D];     // also the fused merge's scratch
    __shared__ float lds_m[NW][HPW], lds_l[NW][HPW], lds_w[NW][HPW], lds_M[HPW];
#pragma unroll
    for (int e = 0; e < EPL; ++e) lds_o[wave][lane * EPL + e] = o[e];
    if (sub == 0) {
        lds_m[wave][grp] = m;
        lds_l[wave][grp] = l;
    }
    __syncthreads();
    if (threadIdx.x < HPW) {
        const int g = threadIdx.x;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_m[w][g]);
        const float Mu = (M == kNegInf) ? 0.f : M;
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float wt = exp2_fast(lds_m[w][g] - Mu);
            lds_w[w][g] = wt;
            lsum = fmaf(wt, lds_l[w][g], lsum);
        }
        lds_M[g] = M;
        const int64_t r = ((int64_t)b * a.Hq + h0 + g) * S + s;
        if constexpr (TAIL) {
            store_partial(a.ws_m + r, M);
            store_partial(a.ws_l + r, lsum);
        } else {
            a.ws_m[r] = M;
            a.ws_l[r] = lsum;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < HPW * D; i += kHeadsThreads) {
        const int g = i / D, e = i % D;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc = fmaf(lds_w[w][g], lds_o[w][i], acc);
        const bool v_head = a.v_scale && (!BLK || !a.v_blk_lg);
        const float vsc = v_head ? a.v_scale[b * a.Hkv + h0 + g] : 1.f;
        const int64_t r = ((int64_t)b * a.Hq + h0 + g) * S + s;
        if constexpr (TAIL) store_partial(a.ws_o + r * D + e, acc * vsc);
        else a.ws_o[r * D + e] = acc * vsc;
    }

    if constexpr (TAIL) {
        static_assert(merge_rows_lds_floats(HPW, kMaxFusedSplits, D) <= NW * HPW * D, "merge scratch fits");
        __shared__ int last;
        int32_t *const cnt = a.cnt + bh;                   // one counter per (b, 4-head group)
        if (arrive_last(cnt, S, &last)) {
            const int64_t row0 = (int64_t)b * a.Hq + h0;   // the group's first workspace row
            float *const ob = a.out + (int64_t)b * a.sob + (int64_t)h0 * a.soh;
            auto out_of = [&](int j) { return ob + (int64_t)j * a.soh; };
            merge_rows<D, kHeadsThreads>(a.ws_m + row0 * S, a.ws_l + row0 * S, a.ws_o + row0 * S * D, S, S, HPW,
                                         out_of, &lds_o[0][0]);
            reset_counter(cnt);
        }
    }
}

// The fused form (a.fused) takes at most kMaxFusedSplits chunks.
bool split_heads_supported(const SplitArgs &a, int d) {
    if ((a.fused && a.S > kMaxFusedSplits) || a.P > 1 || a.group != 1 || a.nq != 1 || a.Hkv < 2 ||
        a.Hq % kHeadsPerWave)
        return false;
    if (d != 64 && d != 128 && d != 256) return false;
    if (a.skh != d || a.svh != d) return false;              // heads of a key adjacent
    return a.skj >= (int64_t)kHeadsPerWave * d && a.svj >= (int64_t)kHeadsPerWave * d;
}

template <int D, int KVT, bool BLK = false>
static hipError_t launch_ht(const SplitArgs &a, hipStream_t st) {
    const int64_t grid = (int64_t)a.B * (a.Hq / kHeadsPerWave) * a.S;
    if (grid <= 0) return hipSuccess;
    if (a.fused && a.S > kMaxFusedSplits) return hipErrorInvalidValue;
    if (a.block_table) {
        if (a.fused)
            hipLaunchKernelGGL((split_heads_kernel<D, KVT, true, true, BLK>), dim3((unsigned)grid),
                               dim3(kHeadsThreads), 0, st, a);
        else
            hipLaunchKernelGGL((split_heads_kernel<D, KVT, true, false, BLK>), dim3((unsigned)grid),
                               dim3(kHeadsThreads), 0, st, a);
    } else {
        if (a.fused)
            hipLaunchKernelGGL((split_heads_kernel<D, KVT, false, true, BLK>), dim3((unsigned)grid),
                               dim3(kHeadsThreads), 0, st, a);
        else
            hipLaunchKernelGGL((split_heads_kernel<D, KVT, false, false, BLK>), dim3((unsigned)grid),
                               dim3(kHeadsThreads), 0, st, a);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_hd(const SplitArgs &a, hipStream_t st) {
    const bool blk = a.k_blk_lg || a.v_blk_lg;         // FP8 block scales: kernels of their own
    switch (a.kv_type) {
        case kKvF32: return launch_ht<D, kKvF32>(a, st);
        case kKvBF16: return launch_ht<D, kKvBF16>(a, st);
        case kKvE4M3: return blk ? launch_ht<D, kKvE4M3, true>(a, st) : launch_ht<D, kKvE4M3>(a, st);
        case kKvE5M2: return blk ? launch_ht<D, kKvE5M2, true>(a, st) : launch_ht<D, kKvE5M2>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_split_heads(const SplitArgs &a, int d, hipStream_t st) {
    switch (d) {
        case 64: return launch_hd<64>(a, st);
        case 128: return launch_hd<128>(a, st);
        case 256: return launch_hd<256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tad
