// combine.hip -- merge step of split-KV decoding as its own kernel.
//
// Work-group (row, g) merges column groups g, g + gridDim.y, ... of one (b, h, query
// token) row's S chunk partials with merge_row (merge.h): the global max, weights
// 2^(m_s - M), fixed-order sums, one divide.  The column groups of a row go to
// separate work-groups, so a row with many chunks (one head cut into hundreds of
// chunks) is merged by many CUs at once.  Calls with many rows merge 4 rows per
// work-group instead (combine_rows_kernel), to the same bits.
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

// Many rows of up to 64 chunks (several query tokens per head): work-group r merges
// rows [R r, R r + R) side by side with merge_rows (merge.h) -- each row to merge_row's
// bits, every o value loaded in one round of 16-byte loads.  1024 rows of 24 chunks
// (d = 128): 4.8 us against 6.8 us for one row per work-group with column groups
// (graph replay); with few rows the column groups' many work-groups are faster (32
// rows of 32 chunks: 3.5 us against 3.9 us with one row per work-group).
// SCAN: the rows' m are read first: chunks past the last one with a finite m in any of
// the R rows are empty (the split kernels write m = -inf there and leave o unwritten),
// and merge_rows takes them as the merge identity without reading their o -- on ragged
// batches about a third to a half of the o a row would otherwise read.  Same bits.  It
// costs a dependent round trip, which pays only on large partial sets: 2048 rows x 24
// chunks (8 query tokens on the ragged grouped-query batches, 25 MB of o), cold steps
// 133.1-133.3 -> 128.8-129.6 us (bf16) and 55.3-55.7 -> 52.2-52.7 us (FP8); 1024 rows
// (13 MB) 46.1-46.4 -> 46.7-46.9 us and 127.1-127.6 -> 127.7-127.9 us.
template <int D, int R, bool SCAN>
__global__ __launch_bounds__(kCombineThreads) void combine_rows_kernel(CombineArgs a) {
    static_assert(R * 64 <= kCombineThreads, "one m per thread");
    __shared__ __align__(16) float lds[merge_rows_lds_floats(R, 64, D)];
    __shared__ int busy_all;
    const int64_t rows = (int64_t)a.B * a.Hq * a.nq;
    const int64_t r0 = (int64_t)blockIdx.x * R;
    const int nr = (int)(rows - r0 < R ? rows - r0 : R);
    const int S = a.S;
    int busy = S;
    if constexpr (SCAN) {
        const int tid = threadIdx.x;
        if (tid == 0) busy_all = 0;
        __syncthreads();
        if (tid < nr * S && a.ws_m[r0 * S + tid] != kNegInf) atomicMax(&busy_all, tid % S + 1);
        __syncthreads();
        busy = busy_all;
    }
    auto out_of = [&](int j) {
        const int64_t row = r0 + j;                // (b * Hq + h) * nq + t
        const int64_t t = row % a.nq, bh = row / a.nq;
        return a.out + (bh / a.Hq) * a.sob + (bh % a.Hq) * a.soh + t * a.sot;
    };
    merge_rows<D, kCombineThreads>(a.ws_m + r0 * S, a.ws_l + r0 * S, a.ws_o + r0 * S * D, S, busy, nr, out_of, lds);
}

template <int D>
static void launch_combine_d(const CombineArgs &a, int64_t rows, hipStream_t st) {
    if (a.S <= 64 && rows >= 1024) {
        const dim3 grid((unsigned)((rows + 3) / 4));
        if (rows * a.S * D >= (int64_t(4) << 20))          // 16 MB of o partials or more
            hipLaunchKernelGGL((combine_rows_kernel<D, 4, true>), grid, dim3(kCombineThreads), 0, st, a);
        else
            hipLaunchKernelGGL((combine_rows_kernel<D, 4, false>), grid, dim3(kCombineThreads), 0, st, a);
        return;
    }
    const dim3 grid((unsigned)rows, (unsigned)merge_column_groups(a.S, D));
    hipLaunchKernelGGL(combine_kernel<D>, grid, dim3(kCombineThreads), 0, st, a);
}

hipError_t launch_combine(const CombineArgs &a, int d, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.nq;
    if (rows <= 0) return hipSuccess;
    switch (d) {
        case 64: launch_combine_d<64>(a, rows, st); break;
        case 128: launch_combine_d<128>(a, rows, st); break;
        case 256: launch_combine_d<256>(a, rows, st); break;
        case 512: launch_combine_d<512>(a, rows, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Pre-merge of chunks read as pieces: work-group r merges chunk r's P piece partials
// into the chunk's (m, l, o) with merge_pieces (merge.h), so that the workspace then
// holds exactly the n_splits chunk partials the caller asked for.  A kernel of its own
// after the split kernel: the pieces' partials are complete and visible when it starts.
// TAIL (a.out non-null, at most kMaxFusedSplits chunks): the chunk partials are written
// through, and the last of a row's S work-groups to arrive (arrive_last) merges the
// row with merge_rows -- the combine's bits -- and returns the counter to zero.
template <int D, bool TAIL>
__global__ __launch_bounds__(kCombineThreads) void pieces_kernel(PiecesArgs a) {
    __shared__ float lds[64 + kCombineThreads];
    const int64_t r = blockIdx.x;                // (row, chunk)
    merge_pieces<D, kCombineThreads, TAIL>(a.sub_m + r * a.P, a.sub_l + r * a.P, a.sub_o + r * a.P * D, a.P,
                                           a.ws_m + r, a.ws_l + r, a.ws_o + r * D, lds);
    if constexpr (TAIL) {
        __shared__ __align__(16) float mlds[merge_rows_lds_floats(1, kMaxFusedSplits, D)];
        __shared__ int last;
        const int64_t row = r / a.S;             // b * Hq + h
        if (arrive_last(a.cnt + row, a.S, &last)) {
            float *const orow = a.out + (row / a.Hq) * a.sob + (row % a.Hq) * a.soh;
            merge_rows<D, kCombineThreads>(a.ws_m + row * a.S, a.ws_l + row * a.S, a.ws_o + row * a.S * D, a.S, a.S, 1,
                                           [&](int) { return orow; }, mlds);
            reset_counter(a.cnt + row);
        }
    }
}

template <int D>
static void launch_pieces_d(const PiecesArgs &a, hipStream_t st) {
    if (a.out)
        hipLaunchKernelGGL((pieces_kernel<D, true>), dim3((unsigned)a.chunks), dim3(kCombineThreads), 0, st, a);
    else
        hipLaunchKernelGGL((pieces_kernel<D, false>), dim3((unsigned)a.chunks), dim3(kCombineThreads), 0, st, a);
}

hipError_t launch_pieces(const PiecesArgs &a, int d, hipStream_t st) {
    if (a.chunks <= 0) return hipSuccess;
    if (a.P < 1 || a.P > 64 || a.P * d > 16384) return hipErrorInvalidValue;
    if (a.out && (a.S < 1 || a.S > kMaxFusedSplits || !a.cnt || a.Hq < 1)) return hipErrorInvalidValue;
    switch (d) {
        case 64: launch_pieces_d<64>(a, st); break;
        case 128: launch_pieces_d<128>(a, st); break;
        case 256: launch_pieces_d<256>(a, st); break;
        case 512: launch_pieces_d<512>(a, st); break;
        default: return hipErrorInvalidValue;
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
