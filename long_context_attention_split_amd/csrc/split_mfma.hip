// split_mfma.hip -- split step for grouped-query attention on the matrix cores (gfx950).
//
// With g query heads sharing one KV head (and/or nq query tokens per head), the
// scores of a key tile form a real dense product S^T[key][column] = K_tile . Q^T over
// the g*nq (head, token) columns, and so does the value update O^T[e][column] +=
// V_tile^T . P^T.  Each wave serves all the columns of one KV head, and the waves of
// a work-group share one (b, chunk) -- 4 waves on one KV head, or 3 (d = 128) or 4
// (d = 64) waves on each of 4 adjacent KV heads -- so every K and V byte of the chunk
// is read from HBM once however many heads and tokens share it.  Each column masks
// the keys past its token's position.  The per-head partials (m, l, o) it writes are
// the same as the vector-ALU kernel's (see split_valu.hip): chunk maximum in base 2,
// sum of 2^(s - m), and the 2^(s - m)-weighted sum of value rows, i.e. the per-chunk
// local max, denominator and numerator of tree_attn_decode ("Tree Attention
// Decoding").
//
// Data path: each wave streams tiles of K and V (16 keys for bf16, 32 keys for FP8:
// 8 KiB at d = 128 either way, 16 KiB at d = 256) straight from HBM into its own LDS
// buffers with
// buffer_load_dwordx4 ... lds.  Every load instruction covers whole consecutive rows
// -- the pattern that streams at full HBM rate -- and the lanes of a row fetch its
// 16-byte chunks in an XOR-swizzled order, so that the matrix-core operand reads
// from LDS hit distinct bank groups.  A wave reads a landed tile's operands into
// registers, issues the next tile's loads into the same buffer, and then computes,
// so the next tile is in flight while the current one is consumed.
//
// Matrix instructions: v_mfma_f32_16x16x32_bf16 (lane l: A[i][k] with i = l%16,
// B[k][j] with j = l%16, k in the 8-wide block l/16; C[i][j] with j = l%16,
// i = 4(l/16) + r) and v_mfma_f32_16x16x16_bf16 (same, 4-wide k blocks).  The
// reduction index only has to be laid out the same way in A and B.
//  * scores: A = 16 keys x 32 dims of K from LDS, B = Q^T with heads on the 16
//    columns (zero past g).  fp32 q is split into bf16 hi + lo and both are
//    multiplied (two MFMAs), keeping ~16 significant bits of q; K is exactly bf16
//    (FP8 K is widened to bf16 in registers, exactly).  Lane l gets the scores of
//    keys 4(l/16)+r of each 16-key block for head l%16.
//  * value update, bf16 (16x16x16): A = V^T (16 value columns x the tile's 16 keys),
//    B = P^T (16 keys x heads), the probabilities split into bf16 hi + lo.  The V^T
//    operand comes straight from the row-major V tile in LDS through gfx950's
//    transposing LDS read (ds_read_b64_tr_b16), one read per 16 value columns.
//  * value update, FP8 (16x16x32 over the 32-key tile): V^T comes from the FP8 tile
//    through the 8-bit transposing read (ds_read_b64_tr_b8), addressed so that each
//    lane's 8 reduction slots are the 8 keys whose probabilities it already holds;
//    it is widened to bf16 in registers.
//
// Work distribution: the (row, KV-head group, chunk) items are numbered busy-first
// (every non-empty chunk of the batch first); work-group i runs busy item i, the grid
// holds at most one work-group per resident slot, and the empty chunks' merge
// identities are written afterwards by single waves.  The chunk length is one per
// batch, lengthened on the device when the non-empty chunks would not fit the
// resident work-groups.  A KV head with more than 16 (head, token) columns (g * nq up
// to 256) has them cut into blocks of 16, the product width.  Each wave runs two
// blocks on every tile it loads (CB = 2: the chunk is read once for 32 columns; FP8
// block-scale kernels keep one); a call with more blocks than that gives each (item,
// group of blocks) a work-group of its own, those of one item on one XCD one after
// another (column_block_of), so that the later ones find the chunk's K and V in its L2.
//
// Softmax per head: lane l owns head l%16 and 4 keys of each 16-key block; the lanes
// l, l^16, l^32, l^48 exchange their max and sum (row swaps, no LDS).  The running
// (m, l) and the rescale of O follow the online softmax of the "Flash Aandacht"
// page's block loop, kept un-normalised, with the reference maximum moved only when
// a column's maximum passes it by more than 2^8 (see below).

#include <type_traits>

#include "device_util.h"
#include "merge.h"
#include "tad_internal.h"

namespace tad {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// x = hi + lo with hi, lo bf16 (truncations): |x - hi - lo| <= 2^-16 |x|.
__device__ __forceinline__ void split_bf16(float x, uint32_t &hi, uint32_t &lo) {
    const uint32_t h = __float_as_uint(x) & 0xffff0000u;
    const float r = x - __uint_as_float(h);              // exact
    hi = h >> 16;
    lo = __float_as_uint(r) >> 16;
}

// Four FP8 codes (one dword) -> four bf16 in two dwords, codes 0, 1 in lo and 2, 3 in
// hi (low half first).  gfx950's scaled conversion with scale 1 is exact: every E4M3
// and E5M2 value is a bf16 number.
template <int KVT>
__device__ __forceinline__ void widen_fp8x4(uint32_t w, uint32_t &lo, uint32_t &hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t a, b;
    if constexpr (KVT == kKvE4M3) {
        a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true);
    } else {
        a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.f, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.f, true);
    }
    lo = __builtin_bit_cast(uint32_t, a);
    hi = __builtin_bit_cast(uint32_t, b);
}

// Reductions over the lanes l, l^16, l^32, l^48 (the four 16-lane rows) with gfx950's
// row swaps, which stay in the VALU (no LDS round trip).  Each swap leaves a lane's own
// value and its partner's in the two results in the same order in both rows of a
// pair, so every lane computes the identical expression.
__device__ __forceinline__ float rows_max(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ f32x4_t mfma16x16x16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// The merge identity (m = -inf, l = 0), written by one wave, for the query columns of
// an empty item: row wi.b, KV heads wi.g * HG .. + HG - 1, chunk wi.s, every column
// block.  Those are the HG * g * nq (head, token) rows R0, R0 + 1, ... of the
// workspace.  The merge gives such a chunk weight 0 and leaves its o out of the sums,
// so o is not written: with 64 rows of d = 128 that is 32 KB per empty item, and on a
// ragged batch of 8 rows with 4 tokens each those stores took about a seventh of the
// kernel's time.
template <int D, int HG>
__device__ __forceinline__ void wave_identity(const SplitArgs &a, const WorkItem wi) {
    const int lane = (int)(threadIdx.x & 63);
    const int rows = HG * a.group * a.nq;
    const int64_t R0 = ((int64_t)wi.b * a.Hq + (int64_t)wi.g * HG * a.group) * a.nq;
    for (int i = lane; i < rows; i += 64) {
        const int64_t r = (R0 + i) * a.S + wi.s;
        a.ws_m[r] = kNegInf;
        a.ws_l[r] = 0.f;
    }
}

// Column blocks: a KV head's g * nq (head, token) columns are cut into blocks of 16, one
// product width, and a work-group serves CB of them; with more, each (busy item, group
// of CB blocks) pair is a work-group of its own that streams the item's K and V.
// Work-group w of the busy ones -> (busy item, block group): the ncb groups of item i
// run on work-groups 8 apart, all on one XCD (the dispatcher sends work-group w to XCD
// w mod 8) and dispatched one after another, so the later ones find the chunk's K and
// V in that XCD's L2; items go in groups of 8, and a last group of fewer items in
// order.  The identity map for ncb = 1.  Wave-uniform.
__device__ __forceinline__ void column_block_of(int w, int busy, int ncb, int *item, int *cb) {
    const int grp = 8 * ncb;
    const int full = busy / 8;                   // complete groups of 8 items
    const int q = w / grp;
    if (q < full) {
        const int r = w - q * grp;
        *item = 8 * q + (r & 7);
        *cb = r >> 3;
    } else {
        const int rem = max(busy - 8 * full, 1); // items of the last group (w < busy * ncb)
        const int j = w - grp * full;
        *item = 8 * full + j % rem;
        *cb = j / rem;
    }
}

// Fused form: the output of the g * nq (head, token) rows of KV head wi.g of row wi.b,
// written as 0 by one wave when the row has no keys -- no chunk of it arrives at a
// counter, so no merge writes it (the merge of such a row gives 0).  Called for the
// row's chunk 0, which is empty exactly then.
template <int D>
__device__ __forceinline__ void wave_zero_rows(const SplitArgs &a, const WorkItem wi) {
    const int lane = (int)(threadIdx.x & 63);
    const int rows = a.group * a.nq;
    for (int i = lane; i < rows * D; i += 64) {
        const int j = i / D, e = i % D;
        a.out[(int64_t)wi.b * a.sob + (int64_t)(wi.g * a.group + j / a.nq) * a.soh + (int64_t)(j % a.nq) * a.sot + e] =
            0.f;
    }
}

// One work item of the matrix-core split kernel: row wi.b, KV heads wi.g * HG ..
// + HG - 1, chunk wi.s of the row's Lb keys cut with chunk length c.  smem and lds_ml
// are the work-group's LDS.
// PAGED: K/V rows come from a paged cache; each 16-row piece of a tile lies inside one
// page (page sizes are multiples of 16) and gets its own buffer resources.
// HG, NWH: a work-group serves HG adjacent KV heads of one chunk with NWH waves each
// (HG = 1: the 4 waves share one KV head).  With HG = 4 and caches that store the KV
// heads of a key next to each other, the waves of the 4 heads read the 4 adjacent
// rows of each key at about the same time, where one head's waves alone would read
// short runs spread over the cache.
// KVT: kKvBF16, or an FP8 format (kKvE4M3, kKvE5M2).  FP8 tiles hold 32 keys (the
// same bytes as a 16-key bf16 tile) and stay FP8 in LDS: the K operands are read
// as they are, the V^T operands through gfx950's 8-bit transposing LDS read
// (ds_read_b64_tr_b8), and both are widened to bf16 in registers (exact: every E4M3
// and E5M2 value is a bf16 number).  The value product then runs on
// v_mfma_f32_16x16x32_bf16 over the 32 keys.  Dequantisation scales per (b, KV head)
// are folded into q (K) and into the wave's O (V); scales per block of key positions
// multiply each 16-key score block (K) and each probability before it becomes the
// value product's operand (V), while l sums the unscaled probabilities.
// WT: the partial is written through to the device coherence point (store_partial),
// for a merge in another work-group of the same launch (the fused form).
// BLK: FP8 K/V with block scales (kernels of their own, so that the per-(b, KV head)
// kernels keep their registers and schedule).
// CB: column blocks per wave (1 or 2); cb: the work-group's first column block is
// cb * CB (16 of the KV head's g * nq columns each, from column 16 cb CB).  With CB = 2
// a wave keeps two blocks' q operands and states and runs both blocks' products on
// each tile it loads, so the chunk's K and V are read once for 32 columns.
// ox: LDS for the merge of blocks 1 .. CB - 1 ((CB - 1) * NW * NB * 64 float4).
template <int D, bool PAGED, int HG, int NWH, int KVT, bool WT = false, bool BLK = false, int CB = 1>
__device__ __forceinline__ void split_mfma_item(const SplitArgs &a, const WorkItem wi, const int cb, const int c,
                                                const int Lb, uint4 *smem, float (*lds_ml)[3][HG * NWH][16],
                                                float4 *ox, int *lds_cnt) {
    static_assert(D == 64 || D == 128 || D == 256, "head dim");
    static_assert(CB == 1 || CB == 2, "column blocks per wave");
    constexpr bool F8 = KVT != kKvBF16;
    static_assert(!BLK || F8, "block scales are for FP8 K/V");
    constexpr int ELEM = F8 ? 1 : 2;     // bytes per K/V element
    constexpr int NKK = D / 32;          // 32-wide slices of d (score reduction)
    constexpr int NB = D / 16;           // 16-wide column blocks of the output
    constexpr int TK = F8 ? 32 : 16;     // keys per wave tile
    constexpr int NSB = TK / 16;         // 16-key score blocks per tile
    constexpr int CH = D * ELEM / 16;    // 16-byte chunks per row
    constexpr int RPI = 64 / CH;         // rows per load instruction
    constexpr int NLD = TK / RPI;        // load instructions per tile and tensor
    constexpr int TILE = TK * CH;        // 16-byte LDS slots per tile and tensor
    constexpr int NW = HG * NWH;         // waves per work-group
    constexpr int THREADS = 64 * NW;
    static_assert(RPI <= 16 && NLD % NSB == 0, "a load instruction stays inside one 16-row piece of a tile");
    static_assert(NB * 64 * 16 <= 2 * TILE * 16, "a wave's O fits in its tile buffers");


    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int c4 = lane >> 4;            // 8-wide (4-wide) reduction block of this lane
    const int j16 = lane & 15;           // column (head) / row (key, value column)

    // Columns of the products are (query head, query token) pairs: product column j16 of
    // block k is the KV head's column jc = 16 (cb CB + k) + j16, which for jc < g*nq is
    // head kvh*g + jc/nq, token jc%nq; with one token this is one head per column.
    const int S = a.S, g = a.group, nq = a.nq;
    const int gq = g * nq;
    const int b = wi.b, s = wi.s;
    const int kvh0 = wi.g * HG;                            // first KV head of the work-group
    const int hx = wave / NWH, wr = wave % NWH;            // this wave's head and rank in it
    const int kvh = kvh0 + hx;
    bool head_ok[CB];
    int tok[CB], h[CB];
#pragma unroll
    for (int k = 0; k < CB; ++k) {
        const int jc = 16 * (cb * CB + k) + j16;
        head_ok[k] = jc < gq;
        tok[k] = head_ok[k] ? jc % nq : 0;
        h[k] = kvh * g + (head_ok[k] ? jc / nq : 0);
    }

    const ChunkRange cr = chunk_of(Lb, s, c);
    const int j0 = cr.j0, j1 = cr.j1;
    const int n = j1 - j0;
    if (n == 0) {                                          // an empty chunk
        if (wave == 0) wave_identity<D, HG>(a, wi);
        return;
    }
    // keys this column's token sees, and that limit relative to the chunk start
    int Lc[CB], lim[CB];
#pragma unroll
    for (int k = 0; k < CB; ++k) {
        Lc[k] = visible_keys(cr.L, nq, tok[k]);
        lim[k] = min(n, Lc[k] - j0);
    }
    // tiles ending at or before lim_all are seen in full by every column
    const int lim_all = __builtin_amdgcn_readfirstlane(min(n, visible_keys(cr.L, nq, 0) - j0));

    const KvRows kvk(a.k, ELEM, a.skb, a.skh, a.skj, a.skp, a, b, kvh);
    const KvRows kvv(a.v, ELEM, a.svb, a.svh, a.svj, a.svp, a, b, kvh);
    const uint32_t krow = kvk.row_bytes, vrow = kvv.row_bytes;
    const __amdgpu_buffer_rsrc_t kr = PAGED ? make_rsrc(nullptr, 0u) : kvk.rows(j0, n);
    const __amdgpu_buffer_rsrc_t vr = PAGED ? make_rsrc(nullptr, 0u) : kvv.rows(j0, n);
    TilePages pages[NSB];                                  // paged: pages of the tiles' 16-row pieces
    int ktile = 0;                                         // paged: tiles issued so far

    // LDS slot (row r, position p) holds chunk p ^ swz(r) of row r.  Within a 16-row
    // score block the 16 rows of an operand read land in distinct 16-byte bank groups
    // (CH = 16 or 32: swz(r) = r, the low 4 bits of the position, since a row is a
    // multiple of the 256-byte bank space; CH = 8: the row parity plus r/2; CH = 4: the
    // row's place in the bank space plus r/4).  Rows 16..31 of an FP8 tile are rotated
    // by CH/2 more, so that the transposing V read, which takes rows from both halves,
    // spreads too.
    constexpr int RD = CH >= 16 ? 1 : 16 / CH;
    auto swz = [](int r) { return (r / RD + (r / 16) * (CH / 2)) % CH; };
    uint4 *const bufA = smem + wave * 2 * TILE;
    const int ld_r = lane / CH, ld_p = lane % CH;
    // A operand of the value product for value columns [16 nb, 16 nb + 16): lane l needs
    // V[4(l/16) + t][16 nb + l%16], t = 0..3.  ds_read_b64_tr_b16 hands lane i of a
    // 16-lane group element i%4 of the 4-element pieces addressed by lanes i/4 + 4t of
    // the group, so lane l addresses row 4(l/16) + (l%16)/4, elements 16 nb + 4(l%4) ..
    // +3 (8 bytes inside one swizzled 16-byte chunk).
    const int tr_row = 4 * c4 + (j16 >> 2);
    auto read_vt = [&](const uint4 *tv, int nb) -> uint2 {
        const int e = 16 * nb + 4 * (lane & 3);
        const uint16_t *p = (const uint16_t *)(tv + tr_row * CH + ((e >> 3) ^ swz(tr_row))) + (e & 7);
        const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p);
        return __builtin_bit_cast(uint2, v);
    };
    // FP8: the A operand of the 16x16x32 value product for value columns [16 nb, +16):
    // lane l needs V[key(8(l/16) + t)][16 nb + l%16], t = 0..7, with reduction slot
    // 8 c + t holding key 4c + t (t < 4) or 16 + 4c + t - 4 (t >= 4) -- the keys whose
    // probabilities the lane already holds.  ds_read_b64_tr_b8 hands lane i of a
    // 16-lane group byte i%8 of the 8-byte pieces addressed by lanes i/8 + 2t, so lane
    // l addresses the row of slot 8 c4 + j16/2, bytes 16 nb + 8 (j16 & 1) .. + 7.
    const int tr8_t = j16 >> 1;
    const int tr8_row = tr8_t < 4 ? 4 * c4 + tr8_t : 16 + 4 * c4 + tr8_t - 4;
    auto read_vt8 = [&](const uint4 *tv, int nb) -> uint2 {
        typedef int v2i_t __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
        const char *p = (const char *)(tv + tr8_row * CH + (nb ^ swz(tr8_row))) + 8 * (j16 & 1);
        return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)p));
    };
    // HBM -> LDS, whole rows per instruction, non-temporal; rows past the chunk end
    // read as zero.
    auto issue_tile = [&](uint4 *tk, int t0) {
        uint4 *tv = tk + TILE;
#pragma unroll
        for (int h = 0; h < NSB; ++h) {                    // 16-row pieces of the tile
            __amdgpu_buffer_rsrc_t krs = kr, vrs = vr;
            int tb = t0;                                   // tile row 0, relative to the resource
            if constexpr (PAGED) {
                const int th = t0 + 16 * h;
                const int nt = max(0, min(16, n - th));
                const int page = pages[h].get(kvk, j0, n, wr * TK + 16 * h, NWH * TK, ktile);
                krs = kvk.page_rows(page, j0 + th, nt);
                vrs = kvv.page_rows(page, j0 + th, nt);
                tb = -16 * h;
            }
#pragma unroll
            for (int u = h * (NLD / NSB); u < (h + 1) * (NLD / NSB); ++u) {
                const int r = u * RPI + ld_r;
                const uint32_t col = 16u * (uint32_t)(ld_p ^ swz(r));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(tk + u * 64), 16,
                                                         (uint32_t)(tb + r) * krow + col, 0, 0, kPolicyNT);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(tv + u * 64), 16,
                                                         (uint32_t)(tb + r) * vrow + col, 0, 0, kPolicyNT);
            }
        }
        if constexpr (PAGED) ++ktile;
    };
    // The first tile's loads go out before q is read, so that their latencies overlap.
    if (wr * TK < n) issue_tile(bufA, wr * TK);

    // ---- B operands of the score product: q of head j16, dims 32kk + 8c4 + t, as hi/lo,
    // scaled into base-2 units and by the K dequantisation scale of the KV head (FP8).
    const bool k_head = F8 && a.k_scale && (!BLK || !a.k_blk_lg);   // one K scale per (b, KV head)
    const bool v_head = F8 && a.v_scale && (!BLK || !a.v_blk_lg);
    const float qs = a.qscale * (k_head ? a.k_scale[b * a.Hkv + kvh] : 1.f);
    const float vs = v_head ? a.v_scale[b * a.Hkv + kvh] : 1.f;   // applied to this wave's O
    uint4 qhi[CB][NKK], qlo[CB][NKK];
#pragma unroll
    for (int k = 0; k < CB; ++k)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        float x[8];
        const int64_t qoff = (int64_t)b * a.sqb + (int64_t)h[k] * a.sqh + (int64_t)tok[k] * a.sqt + 32 * kk + 8 * c4;
        if (a.q_bf16) {
            const uint4 w = *(const uint4 *)((const uint16_t *)a.q + qoff);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(ws[i]); x[2 * i + 1] = bf16_hi(ws[i]); }
        } else {
            const float4 *qp = (const float4 *)((const float *)a.q + qoff);
            const float4 x0 = qp[0], x1 = qp[1];
            x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
            x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
        }
        uint32_t hw[8], lw[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) split_bf16(head_ok[k] ? x[t] * qs : 0.f, hw[t], lw[t]);
        qhi[k][kk] = make_uint4(hw[0] | hw[1] << 16, hw[2] | hw[3] << 16, hw[4] | hw[5] << 16, hw[6] | hw[7] << 16);
        qlo[k][kk] = make_uint4(lw[0] | lw[1] << 16, lw[2] | lw[3] << 16, lw[4] | lw[5] << 16, lw[6] | lw[7] << 16);
    }
    float slope2[CB];
#pragma unroll
    for (int k = 0; k < CB; ++k) slope2[k] = (a.slopes && head_ok[k]) ? a.slopes[h[k]] * 1.4426950408889634f : 0.f;
    const bool alibi = a.slopes != nullptr;

    // Column state: O and l are sums of 2^(s - m) for a reference m that is moved up to
    // the running maximum mx only when mx passes it by more than kSlack (so a tile's
    // weights are at most 2^kSlack and the rescale of O is rare); the epilogue
    // re-expresses every wave's sums against the exact chunk maximum.
    constexpr float kSlack = 8.f;
    float m[CB], mx[CB], l[CB];
    f32x4_t O[CB][NB];
#pragma unroll
    for (int k = 0; k < CB; ++k) {
        m[k] = mx[k] = kNegInf;
        l[k] = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[k][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

    // The matrix operands of one tile, as each lane holds them: K rows for the score
    // product (bf16: 8 dims; FP8: 8 dims of each 16-key block, still FP8), V^T blocks
    // for the value product (bf16: 4 keys; FP8: 8 keys, still FP8).
    struct TileOps {
        typename std::conditional<F8, uint2, uint4>::type k[NSB][NKK];
        uint2 v[NB];
    };
    auto read_tile = [&](const uint4 *tk, TileOps &ops) {
        if constexpr (F8) {
            // dims 32 kk + 8 c4 .. + 7 of row 16 sb + j16: 8 bytes of chunk 2 kk + c4/2
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int r = 16 * sb + j16;
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk)
                    ops.k[sb][kk] = *(const uint2 *)((const uint32_t *)(tk + r * CH + ((2 * kk + (c4 >> 1)) ^ swz(r))) +
                                                     2 * (c4 & 1));
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) ops.v[nb] = read_vt8(tk + TILE, nb);
        } else {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) ops.k[0][kk] = tk[j16 * CH + ((4 * kk + c4) ^ swz(j16))];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) ops.v[nb] = read_vt(tk + TILE, nb);
        }
    };
    auto widen8 = [](uint2 w) -> uint4 {               // 8 FP8 codes -> 8 bf16, in order
        uint4 o;
        widen_fp8x4<KVT>(w.x, o.x, o.y);
        widen_fp8x4<KVT>(w.y, o.z, o.w);
        return o;
    };

    // ALIBI: add the per-head linear bias (wave-uniform: its own loop body).  Only tiles
    // reaching past some column's visible limit run the masking.
    // FP8 block scales of the tile at t0: a 16-key score block lies in one block (blocks
    // hold at least 16 keys; chunks start on block boundaries), so each takes one K and
    // one V scale (scalar loads, issued with the tile's own loads).
    struct TileScales {
        float k[NSB], v[NSB];
    };
    auto load_scales = [&](int t0, TileScales &ts) {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const int jb = __builtin_amdgcn_readfirstlane(j0 + t0 + 16 * sb);
            ts.k[sb] = a.k_blk_lg ? block_scale(a.k_scale, a.k_blk_lg, a.k_nblk, b * a.Hkv + kvh, jb) : 1.f;
            ts.v[sb] = a.v_blk_lg ? block_scale(a.v_scale, a.v_blk_lg, a.v_nblk, b * a.Hkv + kvh, jb) : 1.f;
        }
    };

    auto consume = [&](const TileOps &ops, int t0, const TileScales &ts, auto alibi_c) {
        constexpr bool ALIBI = decltype(alibi_c)::value;
        // scores: p[k][4 sb + r] is key t0 + 16 sb + 4 c4 + r, column j16 of block k; each
        // K operand is widened (FP8) once and serves every block
        float p[CB][4 * NSB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            f32x4_t sh[CB], sl[CB];                        // q hi and lo: independent chains
#pragma unroll
            for (int k = 0; k < CB; ++k) sh[k] = sl[k] = zero4;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                uint4 kop;
                if constexpr (F8) kop = widen8(ops.k[sb][kk]);
                else kop = ops.k[sb][kk];
#pragma unroll
                for (int k = 0; k < CB; ++k) {
                    sh[k] = mfma16x16x32(kop, qhi[k][kk], sh[k]);
                    sl[k] = mfma16x16x32(kop, qlo[k][kk], sl[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < CB; ++k) {
                const f32x4_t sc = sh[k] + sl[k];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = sc[r];
                    if constexpr (BLK) x *= ts.k[sb];
                    if constexpr (ALIBI)
                        x = fmaf(slope2[k], (float)(j0 + t0 + 16 * sb + 4 * c4 + r - (Lc[k] - 1)), x);
                    p[k][4 * sb + r] = x;
                }
            }
        }
        if (t0 + TK > lim_all) {
#pragma unroll
            for (int k = 0; k < CB; ++k)
#pragma unroll
                for (int i = 0; i < 4 * NSB; ++i)
                    p[k][i] = (t0 + 16 * (i / 4) + 4 * c4 + i % 4 < lim[k]) ? p[k][i] : kNegInf;
        }
        // P^T operands per block: reduction slot t of this lane holds p[k][t] -- bf16: key
        // t0 + 4 c4 + t; FP8: the slot order of the V^T read above
        typedef typename std::conditional<F8, uint4, uint2>::type POp;
        POp phi[CB], plo[CB];
#pragma unroll
        for (int k = 0; k < CB; ++k) {
            float mt = p[k][0];
#pragma unroll
            for (int i = 1; i < 4 * NSB; ++i) mt = fmaxf(mt, p[k][i]);
            mt = rows_max(mt);
            mx[k] = fmaxf(mx[k], mt);
            // some column's maximum passed its reference by more than the slack (or its
            // first key arrived): every column's reference moves up to its running maximum
            const bool up = __any(mt > m[k] + kSlack);
            const float m_new = up ? mx[k] : m[k];
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < 4 * NSB; ++i) {
                p[k][i] = exp2_fast(p[k][i] - m_use);
                ps += p[k][i];
            }
            ps = rows_sum(ps);
            if (up) {
                const float alpha = exp2_fast(m[k] - m_use);
                l[k] *= alpha;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) O[k][nb] *= alpha;
            }
            l[k] += ps;
            m[k] = m_new;

            uint32_t ph[4 * NSB], pl[4 * NSB];
#pragma unroll
            for (int i = 0; i < 4 * NSB; ++i) {
                float pv = p[k][i];                    // weight of the value row: V block scale
                if constexpr (BLK) pv *= ts.v[i / 4];
                split_bf16(pv, ph[i], pl[i]);
            }
            if constexpr (F8) {
                phi[k] = make_uint4(ph[0] | ph[1] << 16, ph[2] | ph[3] << 16, ph[4] | ph[5] << 16, ph[6] | ph[7] << 16);
                plo[k] = make_uint4(pl[0] | pl[1] << 16, pl[2] | pl[3] << 16, pl[4] | pl[5] << 16, pl[6] | pl[7] << 16);
            } else {
                phi[k] = make_uint2(ph[0] | ph[1] << 16, ph[2] | ph[3] << 16);
                plo[k] = make_uint2(pl[0] | pl[1] << 16, pl[2] | pl[3] << 16);
            }
        }
        // value products: each V^T operand is widened (FP8) once and serves every block
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (F8) {
                const uint4 vt = widen8(ops.v[nb]);
#pragma unroll
                for (int k = 0; k < CB; ++k) {
                    O[k][nb] = mfma16x16x32(vt, phi[k], O[k][nb]);
                    O[k][nb] = mfma16x16x32(vt, plo[k], O[k][nb]);
                }
            } else {
#pragma unroll
                for (int k = 0; k < CB; ++k) {
                    O[k][nb] = mfma16x16x16(ops.v[nb], phi[k], O[k][nb]);
                    O[k][nb] = mfma16x16x16(ops.v[nb], plo[k], O[k][nb]);
                }
            }
        }
    };

    constexpr int STRIDE = NWH * TK;
    constexpr int VM_ALL = 0x0F70;                 // s_waitcnt vmcnt(0)
    constexpr int LGKM_ALL = 0xC07F;               // s_waitcnt lgkmcnt(0)
    // The buffer is refilled as soon as the tile's operands are in registers (the LDS
    // reads have returned), and the tile is consumed while the next one loads.
    auto run = [&](auto alibi_c) {
        int t0 = wr * TK;                          // its loads were issued above
        TileScales ts, tsn;                        // BLK: scales of this tile and the next
        if constexpr (BLK) load_scales(t0, ts);
        while (t0 < n) {
            __builtin_amdgcn_s_waitcnt(VM_ALL);
            TileOps ops;
            read_tile(bufA, ops);
            __builtin_amdgcn_s_waitcnt(LGKM_ALL);
            const int tn = t0 + STRIDE;
            if (tn < n) {
                issue_tile(bufA, tn);
                if constexpr (BLK) load_scales(tn, tsn);
            }
            consume(ops, t0, ts, alibi_c);
            if constexpr (BLK) ts = tsn;
            t0 = tn;
        }
    };
    if (alibi) run(std::true_type{});
    else run(std::false_type{});

    // ---- merge the NWH wave states of each head.  Waves of rank > 0 put their state in
    // LDS -- O in their own tile buffer, free now, as 16-byte pieces in lane order (no
    // bank conflicts), and (m, l, mx) per column -- and every lane then adds 1 to
    // lds_cnt[hx] with workgroup-scope release, publishing its own stores.  The rank-0
    // wave of the head waits (acquire) until all 64 (NWH - 1) lanes have counted, not
    // for the other heads' waves, merges the states in registers in rank order and
    // stores the partial straight from its registers: per column, M = the largest
    // running maximum, each wave's weight 2^(m_w - M) against its reference maximum m_w,
    // l = sum_w weight_w l_w, o = sum_w weight_w O_w.
    // With CB = 2 the second block's O goes to the wave's piece of ox, and its
    // (m, l, mx) to lds_ml[1].
    auto o_area = [&](int k, int wv) -> float4 * {             // NB * 64 pieces
        return k == 0 ? reinterpret_cast<float4 *>(smem + wv * 2 * TILE) : ox + ((k - 1) * NW + wv) * NB * 64;
    };
    if (wr > 0) {
#pragma unroll
        for (int k = 0; k < CB; ++k) {
            float4 *const mine = o_area(k, wave);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                mine[nb * 64 + lane] = make_float4(O[k][nb][0], O[k][nb][1], O[k][nb][2], O[k][nb][3]);
            if (c4 == 0) {
                lds_ml[k][0][wave][j16] = m[k];
                lds_ml[k][1][wave][j16] = l[k];
                lds_ml[k][2][wave][j16] = mx[k];
            }
        }
        __hip_atomic_fetch_add(&lds_cnt[hx], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        return;
    }
    while (__hip_atomic_load(&lds_cnt[hx], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < 64 * (NWH - 1))
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int k = 0; k < CB; ++k) {
        float M = mx[k];
#pragma unroll
        for (int w = 1; w < NWH; ++w) M = fmaxf(M, lds_ml[k][2][wave + w][j16]);
        const float Mu = (M == kNegInf) ? 0.f : M;
        const float w0 = exp2_fast(m[k] - Mu);
        float lsum = w0 * l[k];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[k][nb] *= w0;
#pragma unroll
        for (int w = 1; w < NWH; ++w) {
            const float wk = exp2_fast(lds_ml[k][0][wave + w][j16] - Mu);
            lsum = fmaf(wk, lds_ml[k][1][wave + w][j16], lsum);
            const float4 *const other = o_area(k, wave + w);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float4 t = other[nb * 64 + lane];
                O[k][nb][0] = fmaf(wk, t.x, O[k][nb][0]);
                O[k][nb][1] = fmaf(wk, t.y, O[k][nb][1]);
                O[k][nb][2] = fmaf(wk, t.z, O[k][nb][2]);
                O[k][nb][3] = fmaf(wk, t.w, O[k][nb][3]);
            }
        }
        // The column again, from the lane index: the prologue's column is not kept live
        // through the loop (one register, which the paged FP8 block-scale kernels do not
        // have).
        int j16e = (int)(threadIdx.x & 15);
        asm volatile("" : "+v"(j16e));
        const int jce = 16 * (cb * CB + k) + j16e;
        if (jce < gq) {
            // column jce is workspace row (b * Hq + kvh * g) * nq + jce; lane (c4, j16)
            // holds elements 16 nb + 4 c4 .. + 3
            const int64_t r = (((int64_t)b * a.Hq + (int64_t)kvh * g) * nq + jce) * S + s;
            float *const orow = a.ws_o + r * D + 4 * c4;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float sc = F8 ? vs : 1.f;
                if constexpr (WT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) store_partial(orow + 16 * nb + i, O[k][nb][i] * sc);
                } else {
                    *reinterpret_cast<float4 *>(orow + 16 * nb) =
                        make_float4(O[k][nb][0] * sc, O[k][nb][1] * sc, O[k][nb][2] * sc, O[k][nb][3] * sc);
                }
            }
            if (c4 == 0) {
                if constexpr (WT) {
                    store_partial(a.ws_m + r, M);
                    store_partial(a.ws_l + r, lsum);
                } else {
                    a.ws_m[r] = M;
                    a.ws_l[r] = lsum;
                }
            }
        }
    }
}

// Items (row b, KV-head group, chunk s) in busy-first order: every non-empty chunk of
// the batch first.  Work-group i < busy runs busy item i, so a ragged batch's busy
// items go to the first work-groups, which the dispatcher spreads over the XCDs in
// turn (work-group i runs on XCD i mod 8).  Empty item e's merge identity is written by
// wave slot (busy * NW + e) mod (grid * NW) (slot = work-group * NW + wave): the waves
// of the work-groups without a busy item first, then, after their busy item, those of
// the others.  The grid holds at most one work-group per resident slot
// when the batch's B * G (row, KV-head group) pairs fit in the slots -- the chunk-length
// fit then leaves at most that many busy items -- and every item otherwise.  Launched
// as work-groups of their own, empty chunks queued behind the busy ones (one 12-wave
// work-group fills a CU's LDS) and each paid the prologue again.
// WAVES: occupancy target (waves per SIMD) the register allocator must meet.
// TAIL (one KV head per work-group): the one-launch form.  The last of a (row, KV head)
// pair's busy chunks to finish merges the pair's g * nq (head, token) rows into out
// with merge_rows, behind the arrival ticket of arrive_last (agent-scope acq_rel), and
// returns the counter to zero; the rows' empty chunks are taken as the merge identity,
// and a row with no keys gets 0 from the wave that writes its chunk 0's identity.  Same
// bits as split + combine.  The partials are written through to the device coherence
// point, which leaves the release little to write back: one row of 32 query heads
// over 8 KV heads, 4096 keys at 32 chunks, 16.2 us with plain stores, 13.1 us written
// through, 12.8 us with a relaxed ticket (graph replay).
// CB: 16-column blocks per wave (2: a work-group serves 32 (head, token) columns of
// each of its KV heads from one read of the chunk).
template <int D, int WAVES, bool PAGED, int HG = 1, int NWH = 4, int KVT = kKvBF16, bool TAIL = false,
          bool BLK = false, int CB = 1>
__global__ __launch_bounds__(64 * HG * NWH) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES)))
void split_mfma_kernel(SplitArgs a) {
    static_assert(!TAIL || (HG == 1 && CB == 1), "the fused merge serves one KV head and 16 columns per work-group");
    constexpr bool F8 = KVT != kKvBF16;
    constexpr int TILE = (F8 ? 32 : 16) * (D * (F8 ? 1 : 2) / 16);   // 16-byte slots per tile and tensor
    constexpr int NW = HG * NWH;
    // Per wave: a (K tile, V tile) pair, reused for the merge (and, with CB = 2, the
    // second block's O in ox).
    __shared__ uint4 smem[NW * 2 * TILE];
    __shared__ float4 ox[CB > 1 ? (CB - 1) * NW * (D / 16) * 64 : 1];
    __shared__ float lds_ml[CB][3][NW][16];
    __shared__ int lds_cnt[HG];                            // lanes of each head's waves done with their loop
    if (threadIdx.x < HG) lds_cnt[threadIdx.x] = 0;
    __syncthreads();

    const int G = a.Hkv / HG;
    // work-group column blocks per KV head: CB blocks of 16 columns each
    const int ncb = (((a.group * a.nq + 15) >> 4) + CB - 1) / CB;
    const int len0 = lane_row_len(a, 0);                   // rows 0..63: one load, reused
    // The fit applies where the launcher capped the grid at the resident slots (B * G *
    // ncb <= slots); with more (row, KV-head group, column block) triples than slots no
    // chunk length fits, and the grid holds every item, so the finest chunking stays.
    const int fit_slots = (int64_t)a.B * G * ncb <= a.wg_slots ? a.wg_slots : 0;
    const int c = fit_chunk_len(a, G * ncb, batch_chunk_len(a, len0), len0, fit_slots);
    const int w = (int)blockIdx.x, grid = (int)gridDim.x;
    WorkItem wi{0, 0, 0};
    int busy, item = w, cb = 0;                            // busy items; this work-group's item and block
    if (ncb > 1) {
        busy = busy_items(a, G, c, len0);
        if (w < busy * ncb) column_block_of(w, busy, ncb, &item, &cb);
    }
    if (a.B <= 64) {
        busy = busy_first_small(a, G, item, c, len0, &wi);
    } else {
        busy = busy_items(a, G, c, len0);
        if (item < busy) wi = busy_first_item(a, G, item, c, len0);
    }
    const int busy_wgs = busy * ncb;
    if (w < busy_wgs) {
        const int Lb = wi.b < 64 ? __builtin_amdgcn_readlane(len0, wi.b) : row_len(a, wi.b);
        split_mfma_item<D, PAGED, HG, NWH, KVT, TAIL, BLK, CB>(a, wi, cb, c, Lb, smem, lds_ml, ox, lds_cnt);
        if constexpr (TAIL) {
            __shared__ int last;
            int32_t *const cnt = a.cnt + (int64_t)wi.b * a.Hkv + wi.g;
            if (arrive_last(cnt, min(ceil_div(Lb, c), a.S), &last)) {
                const int gq = a.group * a.nq;
                const int64_t R0 = ((int64_t)wi.b * a.Hq + (int64_t)wi.g * a.group) * a.nq;   // first workspace row
                float *const ob = a.out + (int64_t)wi.b * a.sob + (int64_t)wi.g * a.group * a.soh;
                auto out_of = [&](int j) { return ob + (int64_t)(j / a.nq) * a.soh + (int64_t)(j % a.nq) * a.sot; };
                merge_rows<D, 64 * NW>(a.ws_m + R0 * a.S, a.ws_l + R0 * a.S, a.ws_o + R0 * a.S * D, a.S,
                                       min(ceil_div(Lb, c), a.S), gq, out_of, reinterpret_cast<float *>(smem));
                reset_counter(cnt);
            }
        }
    }
    const int empties = a.B * G * a.S - busy;
    const int slots = grid * NW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int e0 = ((w * NW + wave - busy_wgs * NW) % slots + slots) % slots;
    if (e0 < empties) {
        if (a.B <= 64) {
            const EmptyItems em(a, G, c, len0);
            for (int e = e0; e < empties; e += slots) {
                const WorkItem ei = em.item(e);
                wave_identity<D, HG>(a, ei);
                if constexpr (TAIL) if (ei.s == 0) wave_zero_rows<D>(a, ei);
            }
        } else {
            for (int e = e0; e < empties; e += slots) {
                const WorkItem ei = busy_first_item(a, G, busy + e, c, len0);
                wave_identity<D, HG>(a, ei);
                if constexpr (TAIL) if (ei.s == 0) wave_zero_rows<D>(a, ei);
            }
        }
    }
}

// Most (head, token) columns per KV head the matrix-core kernel takes (g * nq): 16
// blocks of 16; wider calls run the vector kernel.
constexpr int kMaxMfmaColumns = 256;

bool split_mfma_supported(int d, int kv_type, int group, int nq) {
    return (kv_type == kKvBF16 || kv_type == kKvE4M3 || kv_type == kKvE5M2) && (int64_t)group * nq >= 2 &&
           (int64_t)group * nq <= kMaxMfmaColumns && (d == 64 || d == 128 || d == 256);
}

// Fewest (row, 4-KV-head group, chunk) items for which a work-group serves 4 KV heads;
// below it one KV head per work-group gives 4x the work-groups (one row of 32 query
// heads over 8 KV heads, 4096 keys at 8 chunks: 16 twelve-wave work-groups 20.7 us,
// 64 four-wave ones 12.7 us; two rows of 16384 keys at 4 chunks 152.5 -> 50.9 us; at
// 128 items still 11.3 -> 10.3 us (4096 keys, 64 chunks), 19.6 -> 15.9 us (16384 keys,
// 64 chunks), 13.7 -> 11.7 us (two rows, 32 chunks); about even from 256 items on;
// graph replay).
constexpr int64_t kGroupedHeadsMinItems = 256;

// The 4-KV-heads-per-work-group variant: a KV head count divisible by 4.
bool split_mfma_grouped_heads(const SplitArgs &a, int d) {
    return a.Hkv % 4 == 0 && split_mfma_supported(d, a.kv_type, a.group, a.nq);
}

// Whether a call runs the variant with 4 KV heads per work-group.  Not with two column
// blocks per wave (more than 16 columns at d 64/128): with 2 waves per SIMD the 4-head
// form has only 2 waves per KV head, and one KV head per 4-wave work-group measured
// faster (8 query tokens per row, cold steps: ragged FP8 grouped-query batch 60.5-61.8
// -> 54.5-55.3 us, bf16 134.3-134.4 -> 132.1-132.5 us).  Nor for FP8 K/V stored head
// by head ([B, Hkv, L, d]): its 4 heads' rows lie far apart, and one KV head per
// work-group, three work-groups per CU, measured faster (ragged FP8 batch, cold steps,
// three runs each: one token 41.8-41.9 -> 40.6-41.0 us, 4 tokens 47.2-47.3 -> 45.8-46.8
// us, 64-key block scales 44.7-45.2 -> 42.4-42.6 us).  Nor, stored head by head, for
// bf16 K/V with one query head per KV head (several tokens): 2 and 4 tokens on the
// 32-head 131072-key MHA workload 331.7-333.6 -> 317.5-320.0 us per step, 4 tokens on
// the ALiBi workload 323.0-323.4 -> 318.8-320.2 us; bf16 query-head groups keep it
// (ragged grouped-query batch 117.0-117.4 against 118.4-119.8 us).  Caches with the
// heads of a key adjacent (strides or pages) keep the 4-head form, which reads each
// key's adjacent rows together.
static bool runs_grouped_heads(const SplitArgs &a, int d) {
    return split_mfma_grouped_heads(a, d) && (int64_t)a.B * (a.Hkv / 4) * a.S >= kGroupedHeadsMinItems &&
           (a.group * a.nq <= 16 || d == 256) &&
           ((a.kv_type == kKvBF16 && a.group > 1) || a.block_table || a.skh < a.skj);
}

// Whether the one-launch form (TAIL) serves a call: one KV head per work-group, at most
// 64 chunks, and the merge's weights and thread-row sums of the g * nq rows fit in the
// work-group's tile buffers (4 waves x 2 tiles of 2 d 16-byte slots: 64 d floats).
bool split_mfma_fusable(const SplitArgs &a, int d) {
    if (!split_mfma_supported(d, a.kv_type, a.group, a.nq) || runs_grouped_heads(a, d)) return false;
    if (a.group * a.nq > 16) return false;             // one column block: the merge takes <= 16 rows

    return a.S >= 1 && a.S <= 64 && merge_rows_lds_floats(a.group * a.nq, a.S, d) <= 64 * d;
}

// Launched variants: loads overlapped with compute.  The tile held in registers
// costs d/4 + 8 VGPRs per lane; at d = 128 that needs 3 waves per SIMD (152 VGPRs;
// 4 waves would spill), which measured faster than 4 waves without the overlap
// (grouped-query decode, 8 KV heads, 131072 keys: 87.0 vs 93.8 us).  d = 64 keeps 4,
// d = 256 (q operands and O twice d = 128's) runs 2.
// With a KV head count divisible by 4, a work-group runs 4 KV heads x WAVES waves
// (12 waves at d = 128, 16 at d = 64): one work-group per CU at the usual chunk
// count, all resident at once, and for caches with the heads of a key adjacent the 4
// heads' waves read each key's adjacent rows together.  Ragged grouped-query
// workload, 8 KV heads, 32768 keys: d = 128 126.6 -> 119.5 us on [B, Hkv, L, d] K/V
// and 154.5 -> 120.9 us on [B, L, Hkv, d]; d = 64 57.6 -> 54.5 us and 78.8 -> 56.0 us.
// One launch.  wg_slots = the work-groups of this kernel the device runs at once (its
// occupancy per CU, queried once, times the CU count); the grid is capped there when
// the batch's (row, KV-head group) pairs fit in it.
// grid: every (item, work-group column block); capped as above.
template <int D, int WAVES, bool PAGED, int HG, int NWH, int KVT, bool TAIL = false, bool BLK = false, int CB = 1>
static void launch_k(SplitArgs a, int64_t grid, hipStream_t st) {
    constexpr int THREADS = 64 * HG * NWH;
    static const int per_cu = [] {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &nb, reinterpret_cast<const void *>(&split_mfma_kernel<D, WAVES, PAGED, HG, NWH, KVT, TAIL, BLK, CB>),
                THREADS, 0) != hipSuccess || nb < 1)
            nb = 1;
        return nb;
    }();
    a.wg_slots = a.cus * per_cu;
    const int64_t ncb = ((a.group * a.nq + 15) / 16 + CB - 1) / CB;
    if (a.wg_slots > 0 && (int64_t)a.B * (a.Hkv / HG) * ncb <= a.wg_slots && grid > a.wg_slots) grid = a.wg_slots;
    hipLaunchKernelGGL((split_mfma_kernel<D, WAVES, PAGED, HG, NWH, KVT, TAIL, BLK, CB>), dim3((unsigned)grid),
                       dim3(THREADS), 0, st, a);
}

// CB: 16-column blocks per wave.  Two (more than 16 columns, per-(b, KV head) scales)
// cost 2 x (q operands + O) registers: d = 128 then runs 2 waves per SIMD (8-wave
// work-groups for 4 KV heads), d = 64 3.
template <int D, int KVT, bool BLK = false, int CB = 1>
static void launch_mfma_t(const SplitArgs &a, hipStream_t st) {
    constexpr int WAVES = CB == 1 ? (D == 256 ? 1 : D == 128 ? 3 : 4) : (D == 128 ? 2 : 3);
    const int64_t ncb = ((a.group * a.nq + 15) / 16 + CB - 1) / CB;   // work-group column blocks
    const int64_t items = (int64_t)a.B * a.Hkv * a.S * ncb;
    if constexpr (CB == 1) {
        if (a.fused) {                                 // split_mfma_fusable holds
            if (a.block_table) launch_k<D, WAVES, true, 1, 4, KVT, true, BLK>(a, items, st);
            else launch_k<D, WAVES, false, 1, 4, KVT, true, BLK>(a, items, st);
            return;
        }
    }
    if (runs_grouped_heads(a, D)) {
        constexpr int NWH = WAVES;                         // one work-group fills a CU
        const int64_t grid = (int64_t)a.B * (a.Hkv / 4) * a.S * ncb;
        if (a.block_table) launch_k<D, WAVES, true, 4, NWH, KVT, false, BLK, CB>(a, grid, st);
        else launch_k<D, WAVES, false, 4, NWH, KVT, false, BLK, CB>(a, grid, st);
        return;
    }
    if (a.block_table) launch_k<D, WAVES, true, 1, 4, KVT, false, BLK, CB>(a, items, st);
    else launch_k<D, WAVES, false, 1, 4, KVT, false, BLK, CB>(a, items, st);
}

// Per-(b, KV head) scales and more than 16 columns per KV head: two column blocks per
// wave (d 64 and 128; at d = 256 one block's q and O already take half the registers).
template <int D, int KVT>
static void launch_mfma_cols(const SplitArgs &a, hipStream_t st) {
    if constexpr (D != 256) {
        if (a.group * a.nq > 16) {
            launch_mfma_t<D, KVT, false, 2>(a, st);
            return;
        }
    }
    launch_mfma_t<D, KVT>(a, st);
}

template <int D>
static void launch_mfma_d(const SplitArgs &a, hipStream_t st) {
    const bool blk = a.k_blk_lg || a.v_blk_lg;         // FP8 block scales: kernels of their own
    switch (a.kv_type) {
        case kKvE4M3:
            if (blk) launch_mfma_t<D, kKvE4M3, true>(a, st);
            else launch_mfma_cols<D, kKvE4M3>(a, st);
            break;
        case kKvE5M2:
            if (blk) launch_mfma_t<D, kKvE5M2, true>(a, st);
            else launch_mfma_cols<D, kKvE5M2>(a, st);
            break;
        default: launch_mfma_cols<D, kKvBF16>(a, st); break;
    }
}

hipError_t launch_split_mfma(const SplitArgs &a, int d, hipStream_t st) {
    if ((int64_t)a.B * a.Hkv * a.S <= 0) return hipSuccess;
    if (a.fused && !split_mfma_fusable(a, d)) return hipErrorInvalidValue;
    switch (d) {
        case 64: launch_mfma_d<64>(a, st); break;
        case 128: launch_mfma_d<128>(a, st); break;
        case 256: launch_mfma_d<256>(a, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tad
