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
// 8 KiB at d = 128 either way) straight from HBM into its own LDS buffers with
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
// resident work-groups.
//
// Softmax per head: lane l owns head l%16 and 4 keys of each 16-key block; the lanes
// l, l^16, l^32, l^48 exchange their max and sum (row swaps, no LDS).  The running
// (m, l) and the rescale of O follow the online softmax of the "Flash Aandacht"
// page's block loop, kept un-normalised, with the reference maximum moved only when
// a column's maximum passes it by more than 2^8 (see below).

#include <type_traits>

#include "device_util.h"
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
// an empty item: row wi.b, KV heads wi.g * HG .. + HG - 1, chunk wi.s.  Those are the
// HG * g * nq (head, token) rows R0, R0 + 1, ... of the workspace (at most 64).  The
// merge gives such a chunk weight 0 and leaves its o out of the sums, so o is not
// written: with 64 rows of d = 128 that is 32 KB per empty item, and on a ragged
// batch of 8 rows with 4 tokens each those stores took about a seventh of the
// kernel's time.
template <int D, int HG>
__device__ __forceinline__ void wave_identity(const SplitArgs &a, const WorkItem wi) {
    const int lane = (int)(threadIdx.x & 63);
    const int rows = HG * a.group * a.nq;
    const int64_t R0 = ((int64_t)wi.b * a.Hq + (int64_t)wi.g * HG * a.group) * a.nq;
    if (lane < rows) {
        const int64_t r = (R0 + lane) * a.S + wi.s;
        a.ws_m[r] = kNegInf;
        a.ws_l[r] = 0.f;
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
// v_mfma_f32_16x16x32_bf16 over the 32 keys.
template <int D, bool PAGED, int HG, int NWH, int KVT>
__device__ __forceinline__ void split_mfma_item(const SplitArgs &a, const WorkItem wi, const int c, const int Lb,
                                                uint4 *smem, float (*lds_ml)[HG * NWH][16]) {
    static_assert(D == 64 || D == 128, "head dim");
    constexpr bool F8 = KVT != kKvBF16;
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
    constexpr int MAXG = 16;
    static_assert(RPI <= 16 && NLD % NSB == 0, "a load instruction stays inside one 16-row piece of a tile");
    static_assert(NW * MAXG * D * 4 <= NW * 2 * TILE * 16, "merge area fits in the tile buffers");


    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int c4 = lane >> 4;            // 8-wide (4-wide) reduction block of this lane
    const int j16 = lane & 15;           // column (head) / row (key, value column)

    // Columns of the products are (query head, query token) pairs: column j16 < g*nq is
    // head kvh*g + j16/nq, token j16%nq; with one token this is one head per column.
    const int S = a.S, g = a.group, nq = a.nq;
    const int gq = g * nq;
    const int b = wi.b, s = wi.s;
    const int kvh0 = wi.g * HG;                            // first KV head of the work-group
    const int hx = wave / NWH, wr = wave % NWH;            // this wave's head and rank in it
    const int kvh = kvh0 + hx;
    const bool head_ok = j16 < gq;
    const int tok = head_ok ? j16 % nq : 0;
    const int h = kvh * g + (head_ok ? j16 / nq : 0);

    const ChunkRange cr = chunk_of(Lb, s, c);
    const int j0 = cr.j0, j1 = cr.j1;
    const int n = j1 - j0;
    if (n == 0) {                                          // an empty chunk
        if (wave == 0) wave_identity<D, HG>(a, wi);
        return;
    }
    // keys this column's token sees, and that limit relative to the chunk start
    const int Lc = visible_keys(cr.L, nq, tok);
    const int lim = min(n, Lc - j0);
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
    // (CH = 16: swz(r) = r; CH = 8: the row parity plus r/2; CH = 4: the row's place in
    // the 256-byte bank space plus r/4).  Rows 16..31 of an FP8 tile are rotated by
    // CH/2 more, so that the transposing V read, which takes rows from both halves,
    // spreads too.
    auto swz = [](int r) { return (r / (16 / CH) + (r / 16) * (CH / 2)) % CH; };
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
    const float qs = a.qscale * ((F8 && a.k_scale) ? a.k_scale[b * a.Hkv + kvh] : 1.f);
    const float vs = (F8 && a.v_scale) ? a.v_scale[b * a.Hkv + kvh] : 1.f;   // applied to this wave's O
    uint4 qhi[NKK], qlo[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        float x[8];
        const int64_t qoff = (int64_t)b * a.sqb + (int64_t)h * a.sqh + (int64_t)tok * a.sqt + 32 * kk + 8 * c4;
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
        for (int t = 0; t < 8; ++t) split_bf16(head_ok ? x[t] * qs : 0.f, hw[t], lw[t]);
        qhi[kk] = make_uint4(hw[0] | hw[1] << 16, hw[2] | hw[3] << 16, hw[4] | hw[5] << 16, hw[6] | hw[7] << 16);
        qlo[kk] = make_uint4(lw[0] | lw[1] << 16, lw[2] | lw[3] << 16, lw[4] | lw[5] << 16, lw[6] | lw[7] << 16);
    }
    const float slope2 = (a.slopes && head_ok) ? a.slopes[h] * 1.4426950408889634f : 0.f;
    const bool alibi = a.slopes != nullptr;

    // Column state: O and l are sums of 2^(s - m) for a reference m that is moved up to
    // the running maximum mx only when mx passes it by more than kSlack (so a tile's
    // weights are at most 2^kSlack and the rescale of O is rare); the epilogue
    // re-expresses every wave's sums against the exact chunk maximum.
    constexpr float kSlack = 8.f;
    float m = kNegInf, mx = kNegInf, l = 0.f;
    f32x4_t O[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) O[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
    auto consume = [&](const TileOps &ops, int t0, auto alibi_c) {
        constexpr bool ALIBI = decltype(alibi_c)::value;
        // scores: p[4 sb + r] is key t0 + 16 sb + 4 c4 + r, head j16
        float p[4 * NSB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            f32x4_t sh = zero4, sl = zero4;                // q hi and lo: two independent chains
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                uint4 kop;
                if constexpr (F8) kop = widen8(ops.k[sb][kk]);
                else kop = ops.k[sb][kk];
                sh = mfma16x16x32(kop, qhi[kk], sh);
                sl = mfma16x16x32(kop, qlo[kk], sl);
            }
            const f32x4_t sc = sh + sl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = sc[r];
                if constexpr (ALIBI) x = fmaf(slope2, (float)(j0 + t0 + 16 * sb + 4 * c4 + r - (Lc - 1)), x);
                p[4 * sb + r] = x;
            }
        }
        if (t0 + TK > lim_all) {
#pragma unroll
            for (int i = 0; i < 4 * NSB; ++i) p[i] = (t0 + 16 * (i / 4) + 4 * c4 + i % 4 < lim) ? p[i] : kNegInf;
        }
        float mt = p[0];
#pragma unroll
        for (int i = 1; i < 4 * NSB; ++i) mt = fmaxf(mt, p[i]);
        mt = rows_max(mt);
        mx = fmaxf(mx, mt);
        // some column's maximum passed its reference by more than the slack (or its
        // first key arrived): every column's reference moves up to its running maximum
        const bool up = __any(mt > m + kSlack);
        const float m_new = up ? mx : m;
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4 * NSB; ++i) {
            p[i] = exp2_fast(p[i] - m_use);
            ps += p[i];
        }
        ps = rows_sum(ps);
        if (up) {
            const float alpha = exp2_fast(m - m_use);
            l *= alpha;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) O[nb] *= alpha;
        }
        l += ps;
        m = m_new;

        // P^T operands: reduction slot t of this lane holds p[t] -- bf16: key
        // t0 + 4 c4 + t; FP8: the slot order of the V^T read above
        uint32_t ph[4 * NSB], pl[4 * NSB];
#pragma unroll
        for (int i = 0; i < 4 * NSB; ++i) split_bf16(p[i], ph[i], pl[i]);
        if constexpr (F8) {
            const uint4 phi = make_uint4(ph[0] | ph[1] << 16, ph[2] | ph[3] << 16, ph[4] | ph[5] << 16,
                                         ph[6] | ph[7] << 16);
            const uint4 plo = make_uint4(pl[0] | pl[1] << 16, pl[2] | pl[3] << 16, pl[4] | pl[5] << 16,
                                         pl[6] | pl[7] << 16);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const uint4 vt = widen8(ops.v[nb]);
                O[nb] = mfma16x16x32(vt, phi, O[nb]);
                O[nb] = mfma16x16x32(vt, plo, O[nb]);
            }
        } else {
            const uint2 phi = make_uint2(ph[0] | ph[1] << 16, ph[2] | ph[3] << 16);
            const uint2 plo = make_uint2(pl[0] | pl[1] << 16, pl[2] | pl[3] << 16);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                O[nb] = mfma16x16x16(ops.v[nb], phi, O[nb]);
                O[nb] = mfma16x16x16(ops.v[nb], plo, O[nb]);
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
        while (t0 < n) {
            __builtin_amdgcn_s_waitcnt(VM_ALL);
            TileOps ops;
            read_tile(bufA, ops);
            __builtin_amdgcn_s_waitcnt(LGKM_ALL);
            const int tn = t0 + STRIDE;
            if (tn < n) issue_tile(bufA, tn);
            consume(ops, t0, alibi_c);
            t0 = tn;
        }
    };
    if (alibi) run(std::true_type{});
    else run(std::false_type{});

    // ---- merge the NW wave states per head through LDS (reusing the tile buffers).
    // Each wave's columns are rows of D floats in its own MAXG * D slot; the 16-byte
    // chunk k of row j is stored at chunk k ^ j (j < 16), so that the 16-byte stores of
    // one column block (one per column, rows 512 bytes apart) land in 16 different
    // bank groups, and the merge's reads of a row (64 consecutive floats) too.
    __syncthreads();
    float *const lds_o = reinterpret_cast<float *>(smem);  // [NW][MAXG][D], chunks swizzled per row
    if (head_ok) {
        float *const orow = lds_o + wave * (MAXG * D) + j16 * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) orow[4 * ((4 * nb + c4) ^ j16) + r] = F8 ? O[nb][r] * vs : O[nb][r];
        if (c4 == 0) {
            lds_ml[0][wave][j16] = m;
            lds_ml[1][wave][j16] = l;
            lds_ml[2][wave][j16] = mx;
        }
    }
    __syncthreads();
    // Per column (head x, column hh), one thread: the exact chunk maximum M, each wave's
    // weight 2^(m_w - M) (written over its reference m_w) and the denominator.
    if (threadIdx.x < HG * gq) {
        const int x = threadIdx.x / gq, hh = threadIdx.x % gq;
        float M = kNegInf;
#pragma unroll
        for (int w = x * NWH; w < x * NWH + NWH; ++w) M = fmaxf(M, lds_ml[2][w][hh]);
        const float Mu = (M == kNegInf) ? 0.f : M;
        float lsum = 0.f;
#pragma unroll
        for (int w = x * NWH; w < x * NWH + NWH; ++w) {
            const float sw = exp2_fast(lds_ml[0][w][hh] - Mu);
            lds_ml[0][w][hh] = sw;
            lsum = fmaf(sw, lds_ml[1][w][hh], lsum);
        }
        const int64_t r = (((int64_t)b * a.Hq + (kvh0 + x) * g) * nq + hh) * S + s;   // hh: column
        a.ws_m[r] = M;
        a.ws_l[r] = lsum;
    }
    __syncthreads();
    // Thread t handles element t % D of rows t / D, t / D + THREADS / D, ... (row = x * gq
    // + hh); THREADS is a multiple of D >= 64, so a wave's row is uniform and (x, hh)
    // advance by subtraction instead of a division per row.
    static_assert(THREADS % D == 0, "a thread keeps one element of its rows");
    constexpr int RSTEP = THREADS / D;
    const int e = (int)threadIdx.x % D;
    int row = __builtin_amdgcn_readfirstlane((int)threadIdx.x / D);
    int x = 0, hh = row;
    while (hh >= gq) { hh -= gq; ++x; }
    for (; row < HG * gq; row += RSTEP) {
        float acc = 0.f;
        const int ecol = 4 * ((e >> 2) ^ hh) + (e & 3);         // swizzled position of element e in row hh
#pragma unroll
        for (int w = x * NWH; w < x * NWH + NWH; ++w) acc = fmaf(lds_ml[0][w][hh], lds_o[w * (MAXG * D) + hh * D + ecol], acc);
        const int64_t r = (((int64_t)b * a.Hq + (kvh0 + x) * g) * nq + hh) * S + s;
        a.ws_o[r * D + e] = acc;
        hh += RSTEP;
        while (hh >= gq) { hh -= gq; ++x; }
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
template <int D, int WAVES, bool PAGED, int HG = 1, int NWH = 4, int KVT = kKvBF16>
__global__ __launch_bounds__(64 * HG * NWH) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES)))
void split_mfma_kernel(SplitArgs a) {
    constexpr bool F8 = KVT != kKvBF16;
    constexpr int TILE = (F8 ? 32 : 16) * (D * (F8 ? 1 : 2) / 16);   // 16-byte slots per tile and tensor
    constexpr int NW = HG * NWH;
    // Per wave: a (K tile, V tile) pair, reused for the merge.
    __shared__ uint4 smem[NW * 2 * TILE];
    __shared__ float lds_ml[3][NW][16];

    const int G = a.Hkv / HG;
    const int len0 = lane_row_len(a, 0);                   // rows 0..63: one load, reused
    const int c = fit_chunk_len(a, G, batch_chunk_len(a, len0), len0, a.wg_slots);
    const int busy = busy_items(a, G, c, len0);
    const int w = (int)blockIdx.x, grid = (int)gridDim.x;
    if (w < busy) {
        const WorkItem wi = busy_first_item(a, G, w, c, len0);
        const int Lb = wi.b < 64 ? __builtin_amdgcn_readlane(len0, wi.b) : row_len(a, wi.b);
        split_mfma_item<D, PAGED, HG, NWH, KVT>(a, wi, c, Lb, smem, lds_ml);
    }
    const int empties = a.B * G * a.S - busy;
    const int slots = grid * NW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int e0 = ((w * NW + wave - busy * NW) % slots + slots) % slots;
    if (e0 < empties) {
        if (a.B <= 64) {
            const EmptyItems em(a, G, c, len0);
            for (int e = e0; e < empties; e += slots) wave_identity<D, HG>(a, em.item(e));
        } else {
            for (int e = e0; e < empties; e += slots) wave_identity<D, HG>(a, busy_first_item(a, G, busy + e, c, len0));
        }
    }
}

bool split_mfma_supported(int d, int kv_type, int group, int nq) {
    return (kv_type == kKvBF16 || kv_type == kKvE4M3 || kv_type == kKvE5M2) && group * nq >= 2 &&
           group * nq <= 16 && (d == 64 || d == 128);
}

// The 4-KV-heads-per-work-group variant: a KV head count divisible by 4.
bool split_mfma_grouped_heads(const SplitArgs &a, int d) {
    return a.Hkv % 4 == 0 && split_mfma_supported(d, a.kv_type, a.group, a.nq);
}

// Launched variants: loads overlapped with compute.  The tile held in registers
// costs d/4 + 8 VGPRs per lane; at d = 128 that needs 3 waves per SIMD (152 VGPRs;
// 4 waves would spill), which measured faster than 4 waves without the overlap
// (grouped-query decode, 8 KV heads, 131072 keys: 87.0 vs 93.8 us).  d = 64 keeps 4.
// With a KV head count divisible by 4, a work-group runs 4 KV heads x WAVES waves
// (12 waves at d = 128, 16 at d = 64): one work-group per CU at the usual chunk
// count, all resident at once, and for caches with the heads of a key adjacent the 4
// heads' waves read each key's adjacent rows together.  Ragged grouped-query
// workload, 8 KV heads, 32768 keys: d = 128 126.6 -> 119.5 us on [B, Hkv, L, d] K/V
// and 154.5 -> 120.9 us on [B, L, Hkv, d]; d = 64 57.6 -> 54.5 us and 78.8 -> 56.0 us.
// One launch.  wg_slots = the work-groups of this kernel the device runs at once (its
// occupancy per CU, queried once, times the CU count); the grid is capped there when
// the batch's (row, KV-head group) pairs fit in it.
template <int D, int WAVES, bool PAGED, int HG, int NWH, int KVT>
static void launch_k(SplitArgs a, int64_t grid, hipStream_t st) {
    constexpr int THREADS = 64 * HG * NWH;
    static const int per_cu = [] {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &nb, reinterpret_cast<const void *>(&split_mfma_kernel<D, WAVES, PAGED, HG, NWH, KVT>), THREADS,
                0) != hipSuccess || nb < 1)
            nb = 1;
        return nb;
    }();
    a.wg_slots = a.cus * per_cu;
    if (a.wg_slots > 0 && (int64_t)a.B * (a.Hkv / HG) <= a.wg_slots && grid > a.wg_slots) grid = a.wg_slots;
    hipLaunchKernelGGL((split_mfma_kernel<D, WAVES, PAGED, HG, NWH, KVT>), dim3((unsigned)grid), dim3(THREADS), 0,
                       st, a);
}

template <int D, int KVT>
static void launch_mfma_t(const SplitArgs &a, hipStream_t st) {
    constexpr int WAVES = D == 128 ? 3 : 4;
    if (split_mfma_grouped_heads(a, D)) {
        constexpr int NWH = WAVES;                         // one work-group fills a CU
        const int64_t grid = (int64_t)a.B * (a.Hkv / 4) * a.S;
        if (a.block_table) launch_k<D, WAVES, true, 4, NWH, KVT>(a, grid, st);
        else launch_k<D, WAVES, false, 4, NWH, KVT>(a, grid, st);
        return;
    }
    const int64_t grid = (int64_t)a.B * a.Hkv * a.S;
    if (a.block_table) launch_k<D, WAVES, true, 1, 4, KVT>(a, grid, st);
    else launch_k<D, WAVES, false, 1, 4, KVT>(a, grid, st);
}

template <int D>
static void launch_mfma_d(const SplitArgs &a, hipStream_t st) {
    switch (a.kv_type) {
        case kKvE4M3: launch_mfma_t<D, kKvE4M3>(a, st); break;
        case kKvE5M2: launch_mfma_t<D, kKvE5M2>(a, st); break;
        default: launch_mfma_t<D, kKvBF16>(a, st); break;
    }
}

hipError_t launch_split_mfma(const SplitArgs &a, int d, hipStream_t st) {
    if ((int64_t)a.B * a.Hkv * a.S <= 0) return hipSuccess;
    switch (d) {
        case 64: launch_mfma_d<64>(a, st); break;
        case 128: launch_mfma_d<128>(a, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tad
