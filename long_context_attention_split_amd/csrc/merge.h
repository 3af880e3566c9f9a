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
    const float inv = (ls > 0.f) ? 1.f / ls : 0.f;
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

}  // namespace tad
