// tad_internal.h -- argument blocks shared by the host library and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace tad {

// Everything the split kernels need, by value (lives in the kernel argument segment).
struct SplitArgs {
    const void *q;          // [B, Hq, nq, d], innermost contiguous
    int64_t sqb, sqh, sqt;  // q element strides
    int32_t q_bf16;         // q dtype: 1 = bf16, 0 = fp32
    int32_t nq;             // query tokens per (b, h): the row's last nq positions, causal
    const void *k, *v;      // [B, Hkv, Lmax, d], innermost contiguous
    int32_t kv_type;        // kKvF32, kKvBF16, kKvE4M3, kKvE5M2 (device_util.h)
    const float *k_scale, *v_scale;  // FP8 dequantisation scales, or null (1): [B * Hkv], or
                                     // [B * Hkv * nblk] when the tensor has block scales
    // Block scales: key j of (b, KV head h) has scale k_scale[(b * Hkv + h) * k_nblk +
    // (j >> k_blk_lg)]; k_blk_lg = 0 means one scale per (b, KV head).  Blocks hold at
    // least 16 keys, and chunks and pieces start on block boundaries (align).
    int32_t k_blk_lg, v_blk_lg;
    int32_t k_nblk, v_nblk;
    int32_t align;          // chunk and piece lengths are multiples of this (pages, scale blocks)
    int64_t skb, skh, skj;  // k element strides
    int64_t svb, svh, svj;  // v element strides
    const int32_t *seq_lens;  // [B] or null
    const float *slopes;      // [Hq] or null
    // Paged K/V cache (block_table non-null): k and v are [num_pages, page_size, Hkv, d]
    // with page strides skp / svp, row strides skj / svj and head strides skh / svh;
    // key j of row b lives in page block_table[b * max_pages + j / page_size].
    const int32_t *block_table;
    int32_t max_pages, page_size, num_pages;
    int64_t skp, svp;
    int32_t B, Hq, Hkv, Lmax, S, group;
    int32_t cus;            // compute units of the device
    int32_t wg_slots;       // matrix-core kernel: work-groups the device runs at once (set by its launcher)
    float qscale;           // d^-1/2 * log2(e): scores come out in base-2 units
    float *ws_m, *ws_l, *ws_o;  // partial arrays (see tad.h)
    // Fused merge: when set, the last work-group to finish a row (counted in cnt)
    // merges the row's partials into out.  cnt must be zero on entry and is left zero.
    int32_t fused;
    int32_t *cnt;           // [B * Hq * nq] arrival counters
    float *out;             // [B, Hq, nq, d] fp32
    int64_t sob, soh, sot;  // out element strides
    // Pieces (vector kernel, one query row per KV head): with P > 1 every chunk is read
    // by P work-groups, piece p holding keys [p * cs, (p + 1) * cs) of the chunk (cs =
    // sub_chunk_len), each writing its partial to sub_m, sub_l, sub_o at index
    // (row * S + s) * P + p; pieces_kernel then merges them into the chunk's (m, l, o).
    int32_t P;
    float *sub_m, *sub_l, *sub_o;   // [rows * S * P], the same, [rows * S * P * d]
};

// Pre-merge of the pieces of `chunks` chunks, P pieces each (see SplitArgs).  With out
// non-null (one query row per head), the last chunk of each row to be pre-merged also
// merges the row's S chunk partials into out (arrival counters cnt [rows], zero on
// entry and left zero).
struct PiecesArgs {
    const float *sub_m, *sub_l, *sub_o;
    float *ws_m, *ws_l, *ws_o;
    int64_t chunks;
    int32_t P;
    int32_t S, Hq;
    int32_t *cnt;
    float *out;             // [B, Hq, d] fp32, or null
    int64_t sob, soh;       // out element strides
};

struct CombineArgs {
    const float *ws_m, *ws_l, *ws_o;
    float *out;             // [B, Hq, nq, d] fp32
    int64_t sob, soh, sot;  // out element strides
    int32_t B, Hq, nq, S;
};

// Keys a query token sees: token t of nq sits at position L - nq + t and sees the keys
// up to it, i.e. the first clamp(L - nq + t + 1, 0, L) keys.
__device__ __forceinline__ int visible_keys(int L, int nq, int t) {
    return min(max(L - nq + t + 1, 0), L);
}

// Keys [j0, j1) of batch row b that chunk s covers, and the row's length L.
// Every row of the batch is cut with one chunk length, c = ceil(Lref / S), where
// Lref is the longest (clamped) length in the batch -- Lmax when no lengths are
// given, which makes the chunks those of torch.chunk(S).  Rows shorter than Lref
// end with empty chunks, and every non-empty work-group has the same amount of work.
// Must be called by whole waves (it reduces the lengths across the wave).
struct ChunkRange {
    int L, j0, j1;
};

// Row b's length, clamped to [0, Lmax].
// Inclusive prefix sum / maximum over the 64 lanes of a wave, in registers (DPP):
// shifts by 1, 2, 4 and 8 lanes within each 16-lane row, then row_bcast:15 and
// row_bcast:31 add row 0's total into row 1 and rows 0-1's into rows 2-3.  Lanes
// before a row's start read as 0, so the maximum needs non-negative values.  One
// VALU operation per step where shuffles take an LDS round trip each.  Whole waves.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

__device__ __forceinline__ int wave_incl_max(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
    return x;
}

// Sum and maximum (of non-negative values) over a wave, as scalars.
__device__ __forceinline__ int wave_total(int x) { return __builtin_amdgcn_readlane(wave_incl_scan(x), 63); }
__device__ __forceinline__ int wave_top(int x) { return __builtin_amdgcn_readlane(wave_incl_max(x), 63); }

__device__ __forceinline__ int row_len(const SplitArgs &a, int b) {
    return a.seq_lens ? min(max(a.seq_lens[b], 0), a.Lmax) : a.Lmax;
}

// Row (lane + 64 i)'s length in lane `lane`, for the rows of one 64-row block; 0 past B.
__device__ __forceinline__ int lane_row_len(const SplitArgs &a, int b0) {
    const int bb = b0 + (int)(threadIdx.x & 63);
    return bb < a.B ? row_len(a, bb) : 0;
}

// The batch chunk length c (wave-uniform).  len0 = lane_row_len(a, 0), loaded once by
// the caller and reused (the whole batch when B <= 64).
__device__ __forceinline__ int batch_chunk_len(const SplitArgs &a, int len0) {
    int Lref = a.Lmax;
    if (a.seq_lens) {
        int mx = len0;
        for (int b0 = 64; b0 < a.B; b0 += 64) mx = max(mx, lane_row_len(a, b0));
        Lref = wave_top(mx);
    }
    int c = (Lref + a.S - 1) / a.S;
    if (a.align > 1) c = (c + a.align - 1) / a.align * a.align;   // whole pages and scale blocks
    return c;
}

__device__ __forceinline__ int batch_chunk_len(const SplitArgs &a) {
    return batch_chunk_len(a, a.seq_lens ? lane_row_len(a, 0) : 0);
}

// ceil(x / y) for 0 <= x < 2^31, 0 < y < 2^31, through a correctly rounded double
// division: the quotient is exact when it is an integer and cannot round across one
// otherwise, so this is exact -- a few instructions where a 32-bit integer division by a
// run-time divisor costs several dozen.
__device__ __forceinline__ int ceil_div(int x, int y) {
    return (int)__builtin_ceil((double)x / (double)y);
}

// The chunk length for a kernel whose work-groups each serve G (row, chunk) units of
// work: the finest length the S slots per row allow (c = batch_chunk_len) when its
// non-empty chunks fit in the `slots` work-groups the device runs at once, else a
// longer length that fits, found by a few proportional steps, and failing those one
// chunk per row (the longest row's length).  Chunks then never wait for a second round
// of work-groups, and a ragged batch still spreads over the whole device.  With
// B * G <= slots the busy work-groups G * sum_b ceil(L_b / c) never exceed slots.
// Wave-uniform.
__device__ __forceinline__ int fit_chunk_len(const SplitArgs &a, int G, int c, int len0, int slots) {
    if (c <= 0 || slots <= 0) return c;
    auto busy_of = [&](int cc) {                 // G * sum_b ceil(L_b / cc)
        int n = 0;
        for (int b0 = 0; b0 < a.B; b0 += 64) n += ceil_div(b0 == 0 ? len0 : lane_row_len(a, b0), cc);
        return wave_total(n) * G;
    };
    int busy = busy_of(c);
    if (busy <= slots) return c;
    int mx = len0;
    for (int b0 = 64; b0 < a.B; b0 += 64) mx = max(mx, lane_row_len(a, b0));
    const int Lref = wave_top(mx);
    for (int it = 0; it < 16 && busy > slots && c < Lref; ++it) {
        int cn = (int)__builtin_ceil((double)c * busy / slots);     // busy scales about as 1/c
        if (a.align > 1) cn = ceil_div(cn, a.align) * a.align;
        c = max(min(cn, Lref), c + 1);
        busy = busy_of(c);
    }
    if (busy > slots) c = Lref;
    return c;
}

// Chunk s of a row of L keys cut with chunk length c.
__device__ __forceinline__ ChunkRange chunk_of(int L, int s, int c) {
    ChunkRange r;
    r.L = L;
    r.j0 = (int)min((int64_t)s * c, (int64_t)L);
    r.j1 = min(r.j0 + c, L);
    return r;
}

__device__ __forceinline__ ChunkRange chunk_range(const SplitArgs &a, int b, int s) {
    return chunk_of(row_len(a, b), s, batch_chunk_len(a));
}

// Block scale of key j of the (b, KV head) pair bh = b * Hkv + h (lg = log2 of the block
// length, nblk blocks per pair).  The block index is capped at the last block: keys past
// a row's end are masked, but a tile may still look one up.
__device__ __forceinline__ float block_scale(const float *sc, int lg, int nblk, int bh, int j) {
    return sc[(int64_t)bh * nblk + min(j >> lg, nblk - 1)];
}

// Item k of the B * G * S items (row b, index g < G, chunk s) with chunk length c, in
// busy-first order: every non-empty chunk of the batch ahead of every empty one -- row
// by row, g by g, chunk by chunk among the non-empty ones, then the same among the
// empty ones.  Wave-uniform; must be called by whole waves.
struct WorkItem {
    int b, g, s;
};

// The number of non-empty items, G * sum_b min(ceil(L_b / c), S).  Wave-uniform.
__device__ __forceinline__ int busy_items(const SplitArgs &a, int G, int c, int len0) {
    if (c <= 0) return 0;
    int n = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) n += min(ceil_div(b0 == 0 ? len0 : lane_row_len(a, b0), c), a.S);
    return wave_total(n) * G;
}

// Batches of at most 64 rows (one row per lane): the number of busy items and, for
// k < busy, busy item k (busy_items and busy_first_item from one scan).  len0 =
// lane_row_len(a, 0).  Wave-uniform; whole waves.
__device__ __forceinline__ int busy_first_small(const SplitArgs &a, int G, int k, int c, int len0, WorkItem *wi) {
    const int lane = (int)(threadIdx.x & 63);
    const int nb = (lane < a.B && c > 0) ? min(ceil_div(len0, c), a.S) : 0;   // busy chunks of row `lane`
    const int incl = wave_incl_scan(nb * G);
    const int busy = __builtin_amdgcn_readlane(incl, 63);
    if (k < busy) {
        const uint64_t hit = __ballot(incl > k);
        const int r = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
        const int nr = __builtin_amdgcn_readlane(nb, r);
        const int off = k - (__builtin_amdgcn_readlane(incl, r) - nr * G);
        wi->b = r;
        wi->g = off / nr;
        wi->s = off - wi->g * nr;
    }
    return busy;
}

// The empty items of a batch of at most 64 rows (one row per lane), numbered e = 0, 1,
// ... in the order busy_first_item gives them after the busy ones.  The per-row counts
// and their prefix sum are worked out once; item(e) is then one ballot.  Built and used
// by whole waves.
struct EmptyItems {
    int G, S, nb, cnt, incl;   // per lane: non-empty chunks of the row, its empty items, prefix sum

    __device__ __forceinline__ EmptyItems(const SplitArgs &a, int G_, int c, int len0) : G(G_), S(a.S) {
        const bool row = (int)(threadIdx.x & 63) < a.B;
        nb = c > 0 ? min(ceil_div(len0, c), S) : 0;
        cnt = row ? (S - nb) * G : 0;
        incl = wave_incl_scan(cnt);
    }
    __device__ __forceinline__ WorkItem item(int e) const {
        const uint64_t hit = __ballot(incl > e);
        const int r = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
        const int ne = S - __builtin_amdgcn_readlane(nb, r);          // empty chunks per index g
        const int off = e - (__builtin_amdgcn_readlane(incl, r) - __builtin_amdgcn_readlane(cnt, r));
        WorkItem w;
        w.b = r;
        w.g = off / ne;
        w.s = S - ne + off % ne;
        return w;
    }
};

__device__ __forceinline__ WorkItem busy_first_item(const SplitArgs &a, int G, int k, int c, int len0) {
    const int lane = (int)(threadIdx.x & 63);
    for (int pass = 0; pass < 2; ++pass) {       // 0: non-empty chunks, 1: empty ones
        for (int b0 = 0; b0 < a.B; b0 += 64) {
            const int bb = b0 + lane;
            int cnt = 0;                         // this row's chunks of the pass
            if (bb < a.B) {
                const int L = b0 == 0 ? len0 : row_len(a, bb);
                const int busy = c > 0 ? min(ceil_div(L, c), a.S) : 0;
                cnt = pass == 0 ? busy : a.S - busy;
            }
            const int incl = wave_incl_scan(cnt * G);
            const int tot = __builtin_amdgcn_readlane(incl, 63);
            if (k < tot) {
                const uint64_t hit = __ballot(incl > k);
                const int r = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
                const int nr = __builtin_amdgcn_readlane(cnt, r);
                const int off = k - (__builtin_amdgcn_readlane(incl, r) - nr * G);
                WorkItem w;
                w.b = b0 + r;
                w.g = off / nr;
                w.s = off % nr + (pass == 0 ? 0 : a.S - nr);
                return w;
            }
            k -= tot;
        }
    }
    return WorkItem{0, 0, 0};                    // not reached for k < B * G * S
}
// Rows of one (b, kv head) of K or V: a strided slab, or pages of a paged cache.
struct KvRows {
    const char *base;       // slab: row 0 of the (b, kv head); paged: cache + kv-head offset
    uint32_t row_bytes;
    const int32_t *table;   // paged: this batch row's block-table row, else null
    int page_size, num_pages;
    int64_t page_bytes;

    __device__ __forceinline__ KvRows(const void *t, int elem, int64_t sb, int64_t sh, int64_t sj, int64_t sp,
                                      const SplitArgs &a, int b, int kvh) {
        row_bytes = (uint32_t)(sj * elem);
        if (a.block_table) {
            base = (const char *)t + (int64_t)kvh * sh * elem;
            table = a.block_table + (int64_t)b * a.max_pages;
            page_size = a.page_size;
            num_pages = a.num_pages;
            page_bytes = sp * elem;
        } else {
            base = (const char *)t + ((int64_t)b * sb + (int64_t)kvh * sh) * elem;
            table = nullptr;
            page_size = num_pages = 0;
            page_bytes = 0;
        }
    }
    // Buffer resource over rows [j, j + rows).  Paged: [j, j + rows) must lie in one
    // page; a block-table entry outside [0, num_pages) gives an empty range, so those
    // keys and values read as zero instead of touching memory outside the cache.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rows(int j, int n) const {
        if (!table) return make_rsrc(base + (int64_t)j * row_bytes, (uint32_t)n * row_bytes);
        return page_rows(page_id(j), j, n);
    }
    // Paged: the block-table entry of the page holding row j (j < Lmax).
    __device__ __forceinline__ int page_id(int j) const { return table[j / page_size]; }
    // Paged: resource over rows [j, j + n) of the page with block-table entry `page`.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rows(int page, int j, int n) const {
        if (page < 0 || page >= num_pages) return make_rsrc(base, 0u);
        return make_rsrc(base + (int64_t)page * page_bytes + (int64_t)(j % page_size) * row_bytes,
                         (uint32_t)n * row_bytes);
    }
};

// Block-table entries of one wave's tiles, fetched 64 at a time with one vector load:
// lane i holds the page of the wave's tile 64 q + i, so a tile's page is a register
// read instead of a dependent memory load in front of its K/V loads.  Tile k of the
// wave starts at row first + k * stride of a chunk of n rows starting at key j0;
// get() must be called for k = 0, 1, 2, ... in order, by the whole wave.
struct TilePages {
    int lane_page = -1;
    __device__ __forceinline__ int get(const KvRows &kv, int j0, int n, int first, int stride, int k) {
        if ((k & 63) == 0) {
            const int t = first + (k + (int)(threadIdx.x & 63)) * stride;
            lane_page = t < n ? kv.page_id(j0 + t) : -1;
        }
        return __builtin_amdgcn_readlane(lane_page, k & 63);
    }
};

// Sub-chunk length: chunk length c cut into P pieces (whole pages for a paged cache).
__device__ __forceinline__ int sub_chunk_len(const SplitArgs &a, int c) {
    int cs = (c + a.P - 1) / a.P;
    if (a.align > 1) cs = (cs + a.align - 1) / a.align * a.align;
    return cs;
}

// Workspace carving (same arithmetic as tad_workspace_bytes).
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Sub-chunks: problems with fewer than kSubSplitBelow (row, chunk) pairs may cut every
// chunk into up to max_sub_splits pieces, each its own work-group, to reach about
// kSubSplitTarget work-groups (a chunk count the caller fixed can leave most compute
// units idle: one fp32 d = 512 head of 4096 keys in 8 chunks ran as 8 work-groups).
// At most 64 pieces, and at most 64 partial values per thread in the pre-merge
// (pieces * d / 256): one round of loads.  A pure function of the sizes, so every
// entry point that sees the same call cuts it the same way.
constexpr int64_t kSubSplitBelow = 256;
constexpr int64_t kSubSplitTarget = 512;
// Shortest chunk (K and V bytes per KV head) worth a work-group of its own; the
// automatic chunk count never goes below it either.
constexpr int64_t kMinChunkBytes = 128 << 10;

inline int max_sub_splits(int64_t rows, int64_t S, int64_t d) {
    const int64_t pairs = rows * S;
    if (pairs <= 0 || pairs >= kSubSplitBelow || d <= 0) return 1;
    int64_t P = kSubSplitTarget / pairs;
    const int64_t cap = 16384 / d < 64 ? 16384 / d : 64;
    if (P > cap) P = cap;
    return P < 1 ? 1 : (int)P;
}

// m, l, o (tad.h), then the arrival counters cnt [rows], then, when chunks may be cut
// into pieces, the pieces' partials sub_m, sub_l [rows * S * Pmax] and sub_o
// [rows * S * Pmax * d].
struct WsLayout {
    size_t off_m, off_l, off_o, off_cnt, off_sm, off_sl, off_so, total;
    int Pmax;
};

inline WsLayout ws_layout(int64_t rows, int64_t S, int64_t d) {
    WsLayout w;
    const size_t n = size_t(rows) * size_t(S);
    w.Pmax = max_sub_splits(rows, S, d);
    const size_t np = w.Pmax > 1 ? n * size_t(w.Pmax) : 0;
    w.off_m = 0;
    w.off_l = align256(n * sizeof(float));
    w.off_o = w.off_l + align256(n * sizeof(float));
    w.off_cnt = w.off_o + align256(n * size_t(d) * sizeof(float));
    w.off_sm = w.off_cnt + align256(size_t(rows) * sizeof(int32_t));
    w.off_sl = w.off_sm + align256(np * sizeof(float));
    w.off_so = w.off_sl + align256(np * sizeof(float));
    w.total = w.off_so + align256(np * size_t(d) * sizeof(float));
    return w;
}

// Arrival counters of a workspace (cnt, from off_cnt).
inline int64_t ws_counters(int64_t rows, int64_t, int64_t) { return rows; }

// Launchers (defined next to their kernels).  Return the hipError_t of the launch.
hipError_t launch_split_valu(const SplitArgs &a, int d, hipStream_t s);
bool split_mfma_supported(int d, int kv_type, int group, int nq);
bool split_mfma_grouped_heads(const SplitArgs &a, int d);
bool split_mfma_fusable(const SplitArgs &a, int d);
hipError_t launch_split_mfma(const SplitArgs &a, int d, hipStream_t s);
bool split_heads_supported(const SplitArgs &a, int d);
hipError_t launch_split_heads(const SplitArgs &a, int d, hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, int d, hipStream_t s);
hipError_t launch_pieces(const PiecesArgs &a, int d, hipStream_t s);
hipError_t launch_fill_zero(int32_t *p, int64_t n, hipStream_t s);

// Keys per work-group tile of the VALU split kernel (for tests of the host logic).
constexpr int kSplitThreads = 256;
constexpr int kCombineThreads = 256;
constexpr int kMaxSplits = 4096;
// Chunk counts up to which small problems merge in the vector kernel's last work-group
// per row: one work-group merges the whole row there, which beyond a few chunks costs
// more than the combine kernel's many (one fp32 d = 512 head of 4096 keys: 16 chunks
// 43 vs 38 us, 64 chunks 55 vs 16 us; 32 bf16 heads of 1024 keys: 4 chunks 13.5 vs
// 15.8 us, 8 chunks about even).
constexpr int kMaxFusedSplits = 8;

}  // namespace tad
