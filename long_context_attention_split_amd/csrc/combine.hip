// combine.hip -- merge step of split-KV decoding.
//
// One work-group per (b, h) row merges that row's S chunk partials (m_s, l_s, o_s):
// M = max_s m_s, w_s = 2^(m_s - M), L = sum_s w_s l_s, out = sum_s w_s o_s / L.
// This is the global max / renormalise / sum / divide sequence that tree_attn_decode
// ("Tree Attention Decoding") performs with one max all-reduce and two sum
// all-reduces across machines; here the chunks live in one GPU's memory, so the
// reductions are a max tree and two sum trees inside one work-group.  m is in base 2
// (the split step's scores are in base-2 units), so the renormalising factor
// exp(local_max - global_max) becomes 2^(m_s - M).
//
// All sums run in a fixed order (strided per-thread partial sums, then a fixed
// tree), so the result is bit-reproducible from run to run.

#include "device_util.h"
#include "tad_internal.h"

namespace tad {

template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
    constexpr int NT = kCombineThreads;
    constexpr int NW = NT / 64;
    const int row = blockIdx.x;
    const int S = a.S;
    const int tid = threadIdx.x;
    const float *m = a.ws_m + (int64_t)row * S;
    const float *l = a.ws_l + (int64_t)row * S;
    const float *o = a.ws_o + (int64_t)row * S * D;

    __shared__ float w[kMaxSplits];
    __shared__ float red[NW];
    __shared__ float part[NT];

    constexpr int R = D <= NT ? NT / D : 1;   // thread rows per output element
    constexpr int PRE = 16;                   // o loads issued up front per thread
    float ov[PRE];
    if constexpr (D <= NT) {
        const int e = tid % D, rr = tid / D;
#pragma unroll
        for (int i = 0; i < PRE; ++i) {
            const int s = rr + i * R;
            ov[i] = (s < S) ? o[(int64_t)s * D + e] : 0.f;
        }
    }

    // global max (tree: per-thread strided max, wave butterfly, then the NW waves)
    float mx = kNegInf;
    for (int s = tid; s < S; s += NT) mx = fmaxf(mx, m[s]);
    mx = wave_max(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, red[i]);
    const float Mu = (M == kNegInf) ? 0.f : M;   // every chunk empty: all weights 0

    // renormalising weights, and the denominator L
    float ls = 0.f;
    for (int s = tid; s < S; s += NT) {
        const float ws = exp2_fast(m[s] - Mu);
        w[s] = ws;
        ls = fmaf(ws, l[s], ls);
    }
    ls = wave_sum(ls);
    __syncthreads();                 // red[] reads above are done; w[] is complete
    if ((tid & 63) == 0) red[tid >> 6] = ls;
    __syncthreads();
    float Lsum = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) Lsum += red[i];
    const float inv = (Lsum > 0.f) ? 1.f / Lsum : 0.f;

    // numerator: R thread rows share the splits of each output element.  The first
    // PRE value loads of every thread were issued before the max reduction above (they
    // do not depend on it), so their latency overlaps it.
    if constexpr (D <= NT) {
        const int e = tid % D, rr = tid / D;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < PRE; ++i) {
            const int s = rr + i * R;
            if (s < S) acc = fmaf(w[s], ov[i], acc);
        }
#pragma unroll 8
        for (int s = rr + PRE * R; s < S; s += R) acc = fmaf(w[s], o[(int64_t)s * D + e], acc);
        part[tid] = acc;
        __syncthreads();
        if (tid < D) {
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < R; ++i) sum += part[i * D + tid];
            const int b = row / a.Hq, h = row % a.Hq;
            a.out[(int64_t)b * a.sob + (int64_t)h * a.soh + tid] = sum * inv;
        }
    } else {
        const int b = row / a.Hq, h = row % a.Hq;
        for (int e = tid; e < D; e += NT) {
            float acc = 0.f;
#pragma unroll 8
            for (int s = 0; s < S; ++s) acc = fmaf(w[s], o[(int64_t)s * D + e], acc);
            a.out[(int64_t)b * a.sob + (int64_t)h * a.soh + e] = acc * inv;
        }
    }
}

hipError_t launch_combine(const CombineArgs &a, int d, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.Hq;
    if (rows <= 0) return hipSuccess;
    switch (d) {
        case 64: hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)rows), dim3(kCombineThreads), 0, st, a); break;
        case 128: hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)rows), dim3(kCombineThreads), 0, st, a); break;
        case 256: hipLaunchKernelGGL(combine_kernel<256>, dim3((unsigned)rows), dim3(kCombineThreads), 0, st, a); break;
        case 512: hipLaunchKernelGGL(combine_kernel<512>, dim3((unsigned)rows), dim3(kCombineThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tad
