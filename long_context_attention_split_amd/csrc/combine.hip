// combine.hip -- merge step of split-KV decoding as its own kernel.
//
// Work-group (row, g) merges column groups g, g + gridDim.y, ... of one (b, h, query
// token) row's S chunk partials with merge_row (merge.h): the global max, weights
// 2^(m_s - M), fixed-order sums, one divide.  The column groups of a row go to
// separate work-groups, so a row with many chunks (one head cut into hundreds of
// chunks) is merged by many CUs at once.
// This is the global max / renormalise / sum / divide sequence that tree_attn_decode
// ("Tree Attention Decoding") performs with one max all-reduce and two sum
// all-reduces across machines; here the chunks live in one GPU's memory.  The split
// kernels can run the same merge in their last-arriving work-group instead (one
// launch); this kernel serves tad_combine and very large chunk counts.

#include "merge.h"
#include "tad_internal.h"

namespace tad {

template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
    static_assert(kCombineThreads == kMergeThreads, "merge_row runs on the whole work-group");
    __shared__ float lds[kMaxSplits + kMergeThreads];
    const int row = blockIdx.x;                  // (b * Hq + h) * nq + t
    const int S = a.S;
    const int t = row % a.nq, bh = row / a.nq;
    const int b = bh / a.Hq, h = bh % a.Hq;
    merge_row<D>(a.ws_m + (int64_t)row * S, a.ws_l + (int64_t)row * S, a.ws_o + (int64_t)row * S * D, S,
                 a.out + (int64_t)b * a.sob + (int64_t)h * a.soh + (int64_t)t * a.sot, lds, (int)blockIdx.y,
                 (int)gridDim.y);
}

hipError_t launch_combine(const CombineArgs &a, int d, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.nq;
    if (rows <= 0) return hipSuccess;
    if (d != 64 && d != 128 && d != 256 && d != 512) return hipErrorInvalidValue;
    const dim3 grid((unsigned)rows, (unsigned)merge_column_groups(a.S, d));
    switch (d) {
        case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(kCombineThreads), 0, st, a); break;
        case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(kCombineThreads), 0, st, a); break;
        case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(kCombineThreads), 0, st, a); break;
        default: hipLaunchKernelGGL(combine_kernel<512>, grid, dim3(kCombineThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

// Zero-fill of the workspace's arrival counters (a kernel rather than a memset so that
// it can sit inside a captured graph).
__global__ void fill_zero_kernel(int32_t *p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

hipError_t launch_fill_zero(int32_t *p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace tad
