// merge.h -- the merge of one (b, h) row's chunk partials, shared by the combine
// kernel and by the split kernels' fused tail.
//
// Given the row's S partials (m_s in base 2, l_s, o_s[d]):
//   M = max_s m_s,  w_s = 2^(m_s - M),  L = sum_s w_s l_s,  out = sum_s w_s o_s / L
// -- the global max / renormalise / sum / divide steps that tree_attn_decode ("Tree
// Attention Decoding") performs with one max all-reduce and two sum all-reduces.
// Empty chunks (m = -inf) get weight 0, and a chunk of weight 0 adds nothing to the
// sums whatever its o holds (so a producer need not write o for an empty chunk); a
// row whose chunks are all empty gets out = 0.
// Every sum runs in a fixed order, so the result is bit-reproducible and identical
// whichever kernel performs the merge.
#pragma once

#include "device_util.h"

namespace tad {

// Loads of the partials are per-lane (vector) loads.  COHERENT: read them at the
// device coherence point (agent-scope atomic loads), for partials that other
// work-groups of the same kernel wrote with agent-scope atomic stores.
constexpr int kMergeThreads = 256;

// acc + w * o, or acc unchanged for a weight of 0 (o may then be anything, NaN included).
__device__ __forceinline__ float add_weighted(float w, float o, float acc) {
    return w != 0.f ? fmaf(w, o, acc) : acc;
}

template <bool COHERENT>
__device__ __forceinline__ float load_partial(const float *p) {
    if constexpr (COHERENT)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

// Store of a partial that another work-group of the same kernel will merge: written
// through to the device coherence point (agent-scope atomic store), so neither side
// needs a cache-wide write-back or invalidate.
__device__ __forceinline__ void store_partial(float *p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival ticket of a work-group on a counter shared by `total` work-groups that each
// publish partials for one merge: true in the last one to arrive.  Called by every
// thread of the work-group.  Ordering (HIP's scoped memory model): the barrier puts
// every thread's earlier partial stores before thread 0's agent-scope release in the
// counter update; the last arrival's update acquires at agent scope, so after the
// second barrier every thread of that work-group sees all the other work-groups'
// partials (the counter updates form one release sequence).  `flag` is a word of LDS.
__device__ __forceinline__ bool arrive_last(int32_t *cnt, int total, int *flag) {
    __syncthreads();
    if (threadIdx.x == 0)
        *flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == total - 1;
    __syncthreads();
    return *flag != 0;
}

// Return an arrival counter to zero once its merge is done (the next use is in a later
// kernel, ordered by the stream).
__device__ __forceinline__ void reset_counter(int32_t *cnt) {
    if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Pre-merge of one chunk's P pieces (m_p in base 2, l_p, o_p[D], written by P
// work-groups of the split kernel, read here in a later kernel) into the chunk's own
// partial: M = max_p m_p, w_p = 2^(m_p - M),
// l = sum_p w_p l_p, o = sum_p w_p o_p -- the same rescale-and-sum as the row merge,
// without the division, since the result is a partial again.  Fixed order: each of
// the TPC thread parts of a column sums its pieces p in order, and the parts are added
// in order; l is a wave sum over the pieces.  All P * D values are loaded in one round
// (at most 64 per thread).  Called by all NT threads; `lds` holds 64 + NT floats.
// WT: write the chunk's partial through to the device coherence point (store_partial),
// for a row merge in another work-group of the same kernel.
template <int D, int NT, bool WT = false>
__device__ __forceinline__ void merge_pieces(const float *m, const float *l, const float *o, int P, float *cm,
                                             float *cl, float *co, float *lds) {
    constexpr int TPC = D >= NT ? 1 : NT / D;      // threads per column
    constexpr int CPT = D >= NT ? D / NT : 1;      // columns per thread
    constexpr int PCAP = 16384 / D < 64 ? 16384 / D : 64;   // most pieces (max_sub_splits)
    constexpr int PPT = PCAP / TPC;                // pieces per thread part: CPT * PPT <= 64 loads
    static_assert(NT % 64 == 0 && (TPC == 1 || NT % D == 0), "work-group shape");
    const int tid = threadIdx.x, lane = tid & 63;
    const int part = TPC > 1 ? tid / D : 0;
    const int col0 = TPC > 1 ? tid % D : tid;
    float *w = lds;            // [64] weights
    float *sums = lds + 64;    // [NT] part sums

    // every load up front: this thread's pieces of its columns, then m and l
    float v[CPT][PPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = part * PPT + i;
            v[c][i] = p < P ? o[(int64_t)p * D + col0 + c * NT] : 0.f;
        }
    const float mp = lane < P ? m[lane] : kNegInf;
    const float lp = lane < P ? l[lane] : 0.f;
    const float M = wave_max(mp);
    const float Mu = (M == kNegInf) ? 0.f : M;
    const float wp = lane < P ? exp2_fast(mp - Mu) : 0.f;
    if (tid < 64) w[lane] = wp;
    const float lsum = wave_sum(wp * lp);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = part * PPT + i;
            if (p < P) acc = add_weighted(w[p], v[c][i], acc);
        }
        if constexpr (TPC == 1) {
            if constexpr (WT) store_partial(co + col0 + c * NT, acc);
            else co[col0 + c * NT] = acc;
        } else {
            sums[tid] = acc;
        }
    }
    if constexpr (TPC > 1) {
        __syncthreads();
        if (tid < D) {
            float t = 0.f;
#pragma unroll
            for (int k = 0; k < TPC; ++k) t += sums[k * D + tid];
            if constexpr (WT) store_partial(co + tid, t);
            else co[tid] = t;
        }
    }
    if (tid == 0) {
        if constexpr (WT) {
            store_partial(cm, M);
            store_partial(cl, lsum);
        } else {
            *cm = M;
            *cl = lsum;
        }
    }
}

// 1 / L, or 0 for a row whose chunks are all empty (L = 0).
__device__ __forceinline__ float merge_inverse(float ls) {
    return (ls > 0.f) ? 1.f / ls : 0.f;
}

// Thread rows per output column in the weighted sum over the chunks: row rr of R takes
// the chunks s = rr, rr + R, ... in order and the R row sums are added in order, so the
// bits depend on (S, D) only -- whichever kernel merges, however many work-groups share
// the row's columns.  About 8 chunks per thread row, at least NC / D rows (every
// thread busy), at most 64.
__host__ __device__ constexpr int merge_thread_rows(int S, int D) {
    int r = 1;
    while (r < 64 && r * 8 < S) r *= 2;
    const int min_r = kMergeThreads / D;
    return r > min_r ? r : (min_r > 0 ? min_r : 1);
}

// Column groups of a row: NC / R columns each.
__host__ __device__ constexpr int merge_column_groups(int S, int D) {
    return D / (kMergeThreads / merge_thread_rows(S, D));
}

// Merge of one row, called by all NT threads of a work-group (NT a multiple of 64, at
// least kMergeThreads): column groups g0, g0 + gstep, ... of the output (all of them
// with g0 = 0, gstep = 1).  The arithmetic runs on the first kMergeThreads threads in a
// fixed order, so the result does not depend on the work-group size or on how the
// column groups are shared out; the other threads only join the barriers.  `lds` must
// hold S + kMergeThreads floats.
template <int D, bool COHERENT = false, int NT = kMergeThreads>
__device__ __forceinline__ void merge_row(const float *m, const float *l, const float *o, int S,
                                          float *out_row, float *lds, int g0 = 0, int gstep = 1) {
    constexpr int NC = kMergeThreads;           // threads that compute
    static_assert(NT % 64 == 0 && NT >= NC && (D & (D - 1)) == 0 && D >= 64, "work-group shape");
    const int tid = threadIdx.x, lane = tid & 63;
    float *w = lds;           // [S] weights
    float *part = lds + S;    // [NC] partial sums
    const int R = merge_thread_rows(S, D);
    const int CW = NC / R;                      // columns per group (divides D)
    const int groups = D / CW;
    const int cc = tid % CW, rr = tid / CW;     // this thread's column in a group, thread row

    // One round of loads up front: the first 64 chunks' m and l, and the first PF
    // partial outputs of this thread's first column -- they do not depend on the
    // weights, so they need not wait for them.
    constexpr int PF = 16;
    float pre[PF];
    {
        const int col = g0 * CW + cc;
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int s = rr + i * R;
            pre[i] = (tid < NC && g0 < groups && s < S) ? load_partial<COHERENT>(o + (int64_t)s * D + col) : 0.f;
        }
    }
    const float m0 = lane < S ? load_partial<COHERENT>(m + lane) : kNegInf;
    const float l0 = lane < S ? load_partial<COHERENT>(l + lane) : 0.f;

    // global max: every wave reduces all S (lane-strided, then a wave scan), so every
    // wave holds the same value without a barrier
    float mx = m0;
    for (int s = lane + 64; s < S; s += 64) mx = fmaxf(mx, load_partial<COHERENT>(m + s));
    mx = wave_max(mx);
    const float Mu = (mx == kNegInf) ? 0.f : mx;

    // weights (stored by wave 0) and the denominator (every wave, same order)
    float ls = 0.f;
    if (lane < S) {
        const float ws = exp2_fast(m0 - Mu);
        if (tid < 64) w[lane] = ws;
        ls = fmaf(ws, l0, ls);
    }
    for (int s = lane + 64; s < S; s += 64) {
        const float ws = exp2_fast(load_partial<COHERENT>(m + s) - Mu);
        if (tid < 64) w[s] = ws;
        ls = fmaf(ws, load_partial<COHERENT>(l + s), ls);
    }
    ls = wave_sum(ls);
    const float inv = merge_inverse(ls);
    __syncthreads();

    for (int gi = g0; gi < groups; gi += gstep) {
        const int col = gi * CW + cc;
        if (tid < NC) {
            float acc = 0.f;
            int s = rr;
            if (gi == g0) {
#pragma unroll
                for (int i = 0; i < PF; ++i, s += R)
                    if (s < S) acc = add_weighted(w[s], pre[i], acc);
            }
#pragma unroll 8
            for (; s < S; s += R) acc = add_weighted(w[s], load_partial<COHERENT>(o + (int64_t)s * D + col), acc);
            part[tid] = acc;
        }
        __syncthreads();
        if (tid < CW) {
            float sum = 0.f;
            for (int i = 0; i < R; ++i) sum += part[i * CW + tid];
            out_row[col] = sum * inv;
        }
        __syncthreads();                        // part and (after the last group) lds reusable
    }
}

// LDS floats merge_rows needs for R rows of S chunks at head dim D: the weights [R][S],
// the rows' 1 / L [R], then (from a multiple of 4) the thread-row sums [R][rows][D].
__host__ __device__ constexpr int merge_rows_lds_floats(int R, int S, int D) {
    return (R * S + R + 3) / 4 * 4 + R * merge_thread_rows(S, D) * D;
}

// Merge of R consecutive workspace rows (row j: m + j S, l + j S, o + j S D) by one
// work-group of NT threads, every row to the same bits as merge_row gives it: the
// weights and the denominator from the same lane order (one wave per row), the same
// thread-row sums of the weighted o (thread row rr adds chunks rr, rr + Rt, ... in
// order, Rt = merge_thread_rows(S, D)), then those sums in order, times 1 / L.  Rows are
// merged side by side, so a work-group merging many rows pays the load latency about
// once per round of KU (row, thread row, 4 columns) units per thread instead of once per
// row.  Chunks s >= busy of every row are empty: their m and l are taken as -inf and 0
// (what the merge identity holds) without loading them, and their o, which weight 0
// leaves out of the sums, is not loaded either.  Needs S <= 64, R <= 4 NT / 64 and
// merge_rows_lds_floats(R, S, D) floats of lds; out_of(j) is row j's output.
// Called by all NT threads; plain loads (the caller orders them after the partials'
// stores).
template <int D, int NT, typename OutOf>
__device__ __forceinline__ void merge_rows(const float *m, const float *l, const float *o, int S, int busy, int R,
                                           OutOf out_of, float *lds) {
    constexpr int NWV = NT / 64;                // waves
    constexpr int RPW = 4;                      // rows per wave at most
    constexpr int KU = 2;                       // units per thread and round
    constexpr int QD = D / 4;                   // column quads per row
    static_assert(NT % 64 == 0 && D % 4 == 0, "work-group shape");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Rt = merge_thread_rows(S, D);
    const int SPT = (S + Rt - 1) / Rt;          // chunks per thread row (at most 8 for S <= 64)
    float *const wl = lds;                      // [R][S] weights
    float *const il = lds + R * S;              // [R] 1 / L
    float4 *const part = reinterpret_cast<float4 *>(lds + (R * S + R + 3) / 4 * 4);   // [R][Rt][QD]
    const int U = R * Rt * QD;                  // (row, thread row, quad) units

    // the first round's o loads and every row's m, l -- none depends on another
    auto load_units = [&](int u0, float4 (&v)[KU][8]) {
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int u = u0 + k * NT + tid;
            const int j = u / (Rt * QD), rr = (u / QD) % Rt, q = u % QD;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int s = rr + i * Rt;
                v[k][i] = (u < U && i < SPT && s < busy)
                              ? *reinterpret_cast<const float4 *>(o + ((int64_t)j * S + s) * D + 4 * q)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };
    float4 v[KU][8];
    load_units(0, v);
    float mv[RPW], lv[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int j = wave + i * NWV;
        mv[i] = (j < R && lane < busy) ? m[j * S + lane] : kNegInf;
        lv[i] = (j < R && lane < busy) ? l[j * S + lane] : 0.f;
    }
    // weights and 1 / L of each row: merge_row's arithmetic on one wave
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int j = wave + i * NWV;
        if (j < R) {
            const float mx = wave_max(mv[i]);
            const float Mu = (mx == kNegInf) ? 0.f : mx;
            float ls = 0.f;
            if (lane < S) {
                const float ws = exp2_fast(mv[i] - Mu);
                wl[j * S + lane] = ws;
                ls = fmaf(ws, lv[i], ls);
            }
            ls = wave_sum(ls);
            if (lane == 0) il[j] = merge_inverse(ls);
        }
    }
    __syncthreads();
    // thread-row sums over the chunks, in merge_row's order
    for (int u0 = 0; u0 < U; u0 += KU * NT) {
        if (u0 > 0) load_units(u0, v);
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int u = u0 + k * NT + tid;
            if (u < U) {
                const int j = u / (Rt * QD), rr = (u / QD) % Rt;
                float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int s = rr + i * Rt;
                    if (i < SPT && s < S) {
                        const float w = wl[j * S + s];
                        acc.x = add_weighted(w, v[k][i].x, acc.x);
                        acc.y = add_weighted(w, v[k][i].y, acc.y);
                        acc.z = add_weighted(w, v[k][i].z, acc.z);
                        acc.w = add_weighted(w, v[k][i].w, acc.w);
                    }
                }
                part[u] = acc;
            }
        }
    }
    __syncthreads();
    // the thread-row sums of each column in order, times 1 / L
    for (int u = tid; u < R * QD; u += NT) {
        const int j = u / QD, q = u % QD;
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i = 0; i < Rt; ++i) {
            const float4 p = part[(j * Rt + i) * QD + q];
            sum.x += p.x;
            sum.y += p.y;
            sum.z += p.z;
            sum.w += p.w;
        }
        const float inv = il[j];
        float *const dst = out_of(j) + 4 * q;
        dst[0] = sum.x * inv;
        dst[1] = sum.y * inv;
        dst[2] = sum.z * inv;
        dst[3] = sum.w * inv;
    }
}

}  // namespace tad
