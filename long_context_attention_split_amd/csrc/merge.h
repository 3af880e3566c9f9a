// merge.h -- the merge of one (b, h) row's chunk partials, shared by the combine
// kernel and by the split kernels' fused tail.
//
// Given the row's S partials (m_s in base 2, l_s, o_s[d]):
//   M = max_s m_s,  w_s = 2^(m_s - M),  L = sum_s w_s l_s,  out = sum_s w_s o_s / L
// -- the global max / renormalise / sum / divide steps that tree_attn_decode ("Tree
// Attention Decoding") performs with one max all-reduce and two sum all-reduces.
// Empty chunks (m = -inf) get weight 0; a row whose chunks are all empty gets out = 0.
// Every sum runs in a fixed order, so the result is bit-reproducible and identical
// whichever kernel performs the merge.
#pragma once

#include "device_util.h"

namespace tad {

// Loads of the partials are per-lane (vector) loads.  COHERENT: read them at the
// device coherence point (agent-scope atomic loads), for partials that other
// work-groups of the same kernel wrote with agent-scope atomic stores.
constexpr int kMergeThreads = 256;

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

// Merge of one row, called by all NT threads of a work-group (NT a multiple of 64, at
// least kMergeThreads).  The arithmetic runs on the first kMergeThreads threads in a
// fixed order, so the result does not depend on the work-group size; the others only
// join the barriers.  `lds` must hold S + kMergeThreads floats.
template <int D, bool COHERENT = false, int NT = kMergeThreads>
__device__ __forceinline__ void merge_row(const float *m, const float *l, const float *o, int S,
                                          float *out_row, float *lds) {
    constexpr int NC = kMergeThreads;           // threads that compute
    static_assert(NT % 64 == 0 && NT >= NC && (D > NC || NC % D == 0), "work-group shape");
    const int tid = threadIdx.x, lane = tid & 63;
    float *w = lds;           // [S] weights
    float *part = lds + S;    // [NC] partial sums

    // One round of loads up front: the first 64 chunks' m and l, and (D <= NC) the first
    // PF partial outputs each computing thread will weigh -- the loads do not depend on
    // the weights, so they need not wait for them.
    constexpr int R = D <= NC ? NC / D : 1;     // thread rows sharing each output element
    constexpr int PF = 16;
    const int e = tid % D, rr = tid / D;
    float pre[PF];
    if constexpr (D <= NC) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int s = rr + i * R;
            pre[i] = (tid < NC && s < S) ? load_partial<COHERENT>(o + (int64_t)s * D + e) : 0.f;
        }
    }
    const float m0 = lane < S ? load_partial<COHERENT>(m + lane) : kNegInf;
    const float l0 = lane < S ? load_partial<COHERENT>(l + lane) : 0.f;

    // global max: every wave reduces all S (lane-strided, then a butterfly), so every
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

    if constexpr (D <= NC) {
        if (tid < NC) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int s = rr + i * R;
                if (s < S) acc = fmaf(w[s], pre[i], acc);
            }
#pragma unroll 8
            for (int s = rr + PF * R; s < S; s += R) acc = fmaf(w[s], load_partial<COHERENT>(o + (int64_t)s * D + e), acc);
            part[tid] = acc;
        }
        __syncthreads();
        if (tid < D) {
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < R; ++i) sum += part[i * D + tid];
            out_row[tid] = sum * inv;
        }
    } else if (tid < NC) {
        for (int e = tid; e < D; e += NC) {
            float acc = 0.f;
#pragma unroll 8
            for (int s = 0; s < S; ++s) acc = fmaf(w[s], load_partial<COHERENT>(o + (int64_t)s * D + e), acc);
            out_row[e] = acc * inv;
        }
    }
    __syncthreads();                            // lds may be reused after the return
}

}  // namespace tad
