/*
 * tad.h -- C ABI of libtad: exact single-query attention decoding over a long KV
 * sequence, split into chunks that run on different compute units of one GPU, with
 * the chunks' partial results merged by the log-sum-exp rescaling rule.
 *
 * What the library computes (per batch row b, query head h and query token t):
 *
 *   out[b,h,t,:] = softmax_j( q[b,h,t,:] . k[b,kh,j,:] / sqrt(d) + beta_j ) v[b,kh,j,:]
 *
 * over the keys j < L_t, with kh = floor(h / (Hq / Hkv)) and beta_j the optional
 * ALiBi bias -slope_h * (L_t - 1 - j).  With one query token (the usual decode
 * step) L_t = L_b.  With nq tokens they are the row's last nq positions and token t
 * sees the keys up to its own position: L_t = clamp(L_b - nq + t + 1, 0, L_b)
 * (causal among the new tokens, as when several drafted tokens are verified).
 * Sources: "Tree Attention Decoding" (tree_attn_decode.py gist), functions
 * regular_decode (the definition) and tree_attn_decode (chunk the keys, keep a local
 * max, a sum of exponentials and an exponential-weighted value sum per chunk, then
 * take the global max, rescale and sum); "ALiBi with causal=True unexpected bias?" (llm-foundry issue 186: the causal
 * bias row and passing a per-head vector instead of a full bias matrix);
 * "Flash Aandacht: Revolutie in Transformer Efficientie", section on the mathematics
 * (softmax decomposition and fusion).
 *
 * The split step is tad_split, the merge step tad_combine; tad_decode and
 * tad_decode_ws run both.  All device work is asynchronous on the given stream.
 *
 * Conventions shared by every entry point:
 *  - Tensors are described by tad_tensor: a DEVICE pointer, a dtype, and shape and
 *    strides in ELEMENTS.  The innermost stride must be 1; every row start must be
 *    16-byte aligned (data pointer and outer strides in bytes multiples of 16).
 *  - q   : [B, Hq, d] (one token) or [B, Hq, nq, d] (nq <= 256 tokens), TAD_F32 or
 *          TAD_BF16.
 *  - k, v: [B, Hkv, Lmax, d] or [B, Lmax, d] (then Hkv = 1); same dtype (TAD_F32,
 *          TAD_BF16, TAD_FP8_E4M3 or TAD_FP8_E5M2) and shape; any outer strides (e.g.
 *          a [B, Lmax, Hkv, d] cache viewed as [B, Hkv, Lmax, d]).  Hq must be a
 *          multiple of Hkv.  FP8 tensors may carry dequantisation scales (the
 *          tensor's `scale`; the real value is stored * scale; NULL means 1): with
 *          `scale_block` = 0 one per (b, kv head), device fp32 [B * Hkv], index
 *          b * Hkv + kv_head; with `scale_block` = n > 0 (a power of two, 16 to
 *          65536) one per (b, kv head, block of n consecutive key positions), device
 *          fp32 [B * Hkv * nblk] with nblk = ceil(Lcap / n) (Lcap: Lmax, or
 *          max_pages * page_size for a paged cache), key j using index
 *          (b * Hkv + kv_head) * nblk + j / n.  K and V choose independently.
 *          `scale` must be NULL and `scale_block` 0 for every other tensor.
 *  - out : like q ([B, Hq, d] or [B, Hq, nq, d]), TAD_F32.
 *  - d (head dimension) must be 64, 128, 256 or 512.
 *  - seq_lens: DEVICE int32 [B] or NULL (every row uses Lmax).  Values are clamped
 *    to [0, Lmax] on the device; keys at or beyond L_b are never read.  A row with
 *    L_b = 0 produces out = 0 (so does a token whose position is before the first key).
 *  - alibi_slopes: DEVICE fp32 [Hq] or NULL (no bias).
 *  - n_splits: chunks per (b, head); <= 0 selects tad_auto_splits().  Every row
 *    is cut into contiguous chunks of one length c = ceil(Lref / n_splits), where
 *    Lref is the longest (clamped) sequence length in the batch (Lmax without
 *    seq_lens): torch.chunk(n_splits) when all rows have the same length.  The last
 *    chunk of a row may be shorter; shorter rows end with empty chunks, which
 *    contribute nothing.  The matrix-core kernel (query-head groups or several
 *    tokens, 2..256 (head, token) rows per KV head, bf16 or FP8 K/V, d 64, 128 or 256;
 *    more than 16 such rows are served in blocks of 16, each block of a chunk a
 *    work-group of its own that reads the chunk's K and V) lengthens c when the batch's non-empty
 *    chunks would need more work-groups than the device runs at once, to the shortest
 *    length that fits (decided on the device from the row lengths); for it n_splits
 *    is the finest chunking.  With block scales c is rounded up to whole blocks of
 *    K and V.  (The result does not depend on the chunking; with one chunk length
 *    every non-empty work-group of a ragged batch has the same amount of work.)
 *  - stream: HIP stream (0 = default stream).  All tensors are owned by the caller
 *    and must stay valid until the stream work completes.  The library never frees
 *    caller memory and keeps no state besides a per-device compute-unit count.
 *  - Errors: 0 on success, a negative TAD_E* code otherwise; nothing is launched when
 *    validation fails.  tad_last_error() gives a message (per calling thread).  No
 *    C++ exception crosses the ABI and the library never aborts.  Faults inside a
 *    kernel surface at the caller's next synchronisation, as for any HIP launch.
 */
#ifndef TAD_H
#define TAD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TAD_VERSION 20100 /* major*10000 + minor*100 + patch */

/* FP8 formats are the OCP ones: E4M3 "fn" (no infinities, max 448) and E5M2. */
enum tad_dtype { TAD_F32 = 0, TAD_BF16 = 1, TAD_FP8_E4M3 = 2, TAD_FP8_E5M2 = 3 };

enum tad_status {
    TAD_OK = 0,
    TAD_EINVAL = -1,       /* null pointer, bad rank, shape mismatch, bad n_splits */
    TAD_EDTYPE = -2,       /* dtype not allowed for this argument */
    TAD_ELAYOUT = -3,      /* innermost stride != 1 or a row not 16-byte aligned */
    TAD_EUNSUPPORTED = -4, /* head dimension or size outside what the kernels handle */
    TAD_EWORKSPACE = -5,   /* workspace missing or too small */
    TAD_EHIP = -6          /* a HIP runtime call or launch failed (message has the reason) */
};

typedef struct tad_tensor {
    void *data;         /* device pointer */
    int32_t dtype;      /* enum tad_dtype */
    int32_t ndim;       /* 3 or 4 */
    int64_t shape[4];
    int64_t stride[4];  /* elements */
    const float *scale; /* FP8 k/v only: device fp32 dequantisation scales, or NULL
                           (a field beyond data/dtype/ndim/shape/stride because FP8 K/V need a
                           per-(b, KV head) scale, folded into q and into the partials) */
    int32_t scale_block; /* FP8 k/v only: 0 = one scale per (b, KV head); n = one per block
                            of n key positions (a power of two, 16..65536; the per-block
                            form applies each key's scale to its score and value weight) */
} tad_tensor;

/* Library version, TAD_VERSION of the build. */
int tad_version(void);

/* Message describing the last error returned on the calling thread ("" if none). */
const char *tad_last_error(void);

/*
 * Chunks per (b, head) chosen when n_splits <= 0, for a batch of B rows with Hq query
 * heads over Hkv KV heads, nq query tokens, Lmax keys, head dimension d and K/V dtype
 * kv_dtype on `device` (-1: the current device): ceil(4 * CUs / (B * Hkv)) for one
 * row, i.e. four (row, KV head, chunk) units per compute unit, and
 * ceil(6 * CUs / (B * Hkv)) for several rows, whose lengths may differ (seq_lens), so
 * that a ragged batch's non-empty chunks still cover the device; but no chunk under
 * 128 KiB of K and V per KV head -- or 32 KiB per KV head for grouped-query calls on the
 * matrix-core kernel (bf16 or FP8 K/V, d 64, 128 or 256, 2..256 (head, token) rows per KV head) with
 * Hkv a multiple of 4 and at most 16 such rows (any number at d = 256), which it serves
 * 4 KV heads to a work-group when there are at least 256 (row, 4-KV-head group, chunk)
 * items and K/V store the KV heads of a key next to each other or are bf16 with
 * query-head groups -- and at least one.  (The count sees no strides: FP8 K/V, and bf16
 * with one query head per KV head, stored head by head get the 32 KiB minimum though
 * their kernel serves one KV head per work-group.)  Returns the
 * count (>= 1) or a negative TAD_E* code (TAD_EINVAL for sizes, TAD_EUNSUPPORTED for
 * d, TAD_EDTYPE for kv_dtype).  (Hq, nq, d and kv_dtype are arguments because the count
 * mirrors the kernel choice and the byte-sized minimum chunk, which depend on them.)
 */
int32_t tad_auto_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t nq, int64_t Lmax, int32_t d, int32_t kv_dtype,
                        int32_t device);

/*
 * Bytes of device workspace tad_decode_ws / tad_split / tad_combine need for
 * B * Hq * nq rows, n_splits chunks and head dimension d (0 if an argument is < 1).
 * (nq is an argument because every query token has its own partials.)
 * Layout (each array starting at a 256-byte boundary), with row = (b * Hq + h) * nq
 * + t and r = row * n_splits + s:
 *     m[r]        fp32: chunk maximum of the scores, in base-2 units (score * log2 e);
 *                 -inf for an empty chunk
 *     l[r]        fp32: sum over the chunk of 2^(score*log2 e - m[r])
 *     o[r * d + e] fp32: sum over the chunk of 2^(score*log2 e - m[r]) * v[., e];
 *                 left unwritten for an empty chunk (tad_combine ignores the o of a
 *                 chunk whose weight is 0, whatever it holds)
 *     cnt[row]    int32: arrival counters of the fused merge (see tad_decode_ws; the
 *                 matrix-core form uses the first B * Hkv, one per (b, KV head), the
 *                 head-packed form the first B * Hq / 4)
 *     sub_m, sub_l, sub_o: when B * Hq * nq * n_splits < 256, the partials of up to
 *                 Pmax = min(512 / (B * Hq * nq * n_splits), 16384 / d, 64) pieces per
 *                 chunk, same meaning as m, l, o for a piece of the chunk
 * m, l, o are the per-chunk (local max, denominator, numerator) of tree_attn_decode,
 * with the maximum kept in base 2.
 *
 * Pieces.  A call with few (row, chunk) pairs would leave most compute units idle
 * (one head cut into 8 chunks is 8 work-groups), so where the vector kernel serves one
 * query row per KV head, each chunk of at least 256 KiB of K+V is read by up to Pmax
 * work-groups, each a contiguous piece of ceil(c / P) keys (whole pages for a paged
 * cache, whole scale blocks with block scales) with P = min(Pmax, chunk bytes /
 * 128 KiB); a second kernel then merges each chunk's pieces into the chunk's (m, l, o)
 * by the same rescale-and-sum.  The chunks
 * themselves, and so the partials tad_split reports, are those n_splits asks for; only
 * their rounding differs from an uncut chunk.  P depends on the call's sizes only, so
 * every entry point cuts a call the same way.
 */
size_t tad_workspace_bytes(int32_t B, int32_t Hq, int32_t nq, int32_t n_splits, int32_t d);

/*
 * Zero a workspace (all ws_bytes of it) with a small kernel on `stream` (no memset, so
 * it may be captured in a graph).  A zeroed workspace is ready for tad_decode_ws.
 */
int tad_workspace_clear(void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Split step: every (b, query head, chunk) partial (m, l, o) into `ws` (layout above).
 * n_splits must be >= 1 here (use tad_auto_splits to pick one).  `ws` is a device
 * buffer of at least tad_workspace_bytes(B, Hq, nq, n_splits, d) bytes, 256-byte aligned.
 * Chunks read as pieces (above) take a second launch that merges them.
 */
int tad_split(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v,
              const int32_t *seq_lens, const float *alibi_slopes, int32_t n_splits,
              void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Merge step: for each (b, h, t) row, M = max_s m, w_s = 2^(m_s - M), L = sum_s w_s
 * l_s, out = sum_s w_s o_s / L, summed in a fixed order (bit-reproducible).  Rows
 * whose chunks are all empty get out = 0.  `out` is fp32 [B, Hq, d] (nq = 1) or
 * [B, Hq, nq, d].  An empty chunk must hold m = -inf (as tad_split writes it): its o is
 * never read with a nonzero weight, and with 16 MB of o or more (many (head, token)
 * rows, at most 64 chunks) the merge reads the rows' m first and skips the o of
 * chunks past each group of 4 rows' last non-empty one.
 */
int tad_combine(const void *ws, size_t ws_bytes, int32_t B, int32_t Hq, int32_t nq, int32_t n_splits,
                int32_t d, tad_tensor *out, hipStream_t stream);

/*
 * Split + merge with a caller-provided workspace (no allocation).  Small problems run
 * as ONE launch, the merge done by the split kernel itself: each work-group writes its
 * partial, and the last one to finish (counted in the workspace's cnt array with
 * agent-scope acquire-release updates) merges, then returns its counter to zero.  Three
 * kernels do this:
 *   - the vector kernel (one query head per work-group: MHA on [B, Hkv, L, d] caches,
 *     and the cases the matrix-core kernel does not take -- fp32 K/V, d 512, more
 *     than 256 (head, token) rows per KV head), when B * Hq * nq * n_splits is below the
 *     device's compute-unit count, n_splits <= 8 and no chunk is cut into pieces: the
 *     last work-group of a row merges the row;
 *   - the matrix-core kernel (grouped-query heads, several tokens), when it serves one
 *     KV head per work-group with at most 16 (head, token) rows, n_splits <= 8,
 *     B * Hkv * n_splits is at most the
 *     compute-unit count and the merge fits the work-group's LDS (all cases but d = 64
 *     with 16 (head, token) rows per KV head): the last work-group of a (b, KV head)
 *     merges that KV head's (head, token) rows side by side;
 *   - the head-packed kernel (caches whose KV heads are interleaved per key, one query
 *     head per KV head), when n_splits <= 8 and B * Hq / 4 * n_splits is at most the
 *     compute-unit count: the last work-group of a (b, 4-head group) merges its 4 rows.
 * Chunks read as pieces (below) on such small grids take two launches: the pieces
 * kernel's last work-group per row merges the row.  Larger problems run the split
 * (and pieces) and combine kernels back to back (the counters are then unused).
 * Either way the output is bit-identical to tad_split followed by tad_combine.  The
 * one-launch form saves a launch where the host's launch rate sets the pace; replayed
 * in a graph it is about as fast as the two kernels, or up to about a microsecond
 * slower.  The counters must be zero the first time a workspace is used
 * (tad_workspace_clear, or memory allocated zeroed); every call that runs to
 * completion leaves them zero, so a workspace can be reused call after call.  Calls
 * that share one workspace must not overlap.
 */
int tad_decode_ws(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v,
                  const int32_t *seq_lens, const float *alibi_slopes, int32_t n_splits,
                  tad_tensor *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Split + merge; the workspace is taken with hipMallocAsync, its counters cleared by
 * a kernel, and it is released with hipFreeAsync on `stream` (stream-ordered, so
 * concurrent calls on different streams do not share it).
 */
int tad_decode(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v,
               const int32_t *seq_lens, const float *alibi_slopes, int32_t n_splits,
               tad_tensor *out, hipStream_t stream);

/*
 * Split + merge without a workspace argument and without allocating: for callers that
 * cannot allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid it).  Arguments, result and errors as tad_decode; the output
 * is bit-identical to tad_decode_ws with the same n_splits.  The partials and counters
 * live in a 16 MiB device array inside the library, one copy per device, held until
 * the process ends; its counters are cleared by a kernel on `stream` at the first call
 * on a device.  A call whose partials need more than 16 MiB - 256 KiB
 * (tad_workspace_bytes) or more than 65536 counters fails with TAD_EWORKSPACE before
 * anything is launched.  Every call on a device shares that array: calls that overlap
 * on one device (different streams without ordering between them, or host threads)
 * race and give wrong results.
 */
int tad_decode_noalloc(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v,
                       const int32_t *seq_lens, const float *alibi_slopes, int32_t n_splits,
                       tad_tensor *out, hipStream_t stream);

/*
 * Paged K/V cache.  The pages leave the K/V cache to the caller (SwitchHead README,
 * forward signature: the caller keeps the cache and hands it back each step); a
 * paged cache is the layout serving engines use for it: a shared pool of
 * fixed-size pages, each sequence owning a list of pages in a block table.  This
 * layout is not on the pages; it only changes where key j of row b is read:
 * page block_table[b * max_pages + j / page_size], row j % page_size of that page.
 *  - k_cache, v_cache: 4-D [num_pages, page_size, Hkv, d], same dtype and shape,
 *    TAD_BF16, TAD_FP8_E4M3 or TAD_FP8_E5M2 (FP8 with the `scale` and `scale_block`
 *    described above, blocks counted in logical key positions); innermost stride 1,
 *    any outer strides, rows 16-byte aligned;
 *    page_size a multiple of 16; d 64, 128 or 256.
 *  - pages->block_table: DEVICE int32 [B, max_pages], row-major, pages->max_pages
 *    >= 1.  The logical length is Lmax = max_pages * page_size; only the entries
 *    covering the first L_b keys of row b are read.  An entry outside [0, num_pages)
 *    is not checked on the host (the table lives on the device): its keys and
 *    values read as zeros, and no memory outside the cache is touched.
 *  - The chunk length c = ceil(Lref / n_splits) is rounded up to whole pages (and
 *    scale blocks).
 * q, out, seq_lens, alibi_slopes, n_splits, the workspace and the error codes are
 * as for tad_split / tad_decode_ws / tad_decode; the result equals theirs on the
 * gathered [B, Hkv, Lmax, d] K and V up to rounding (the chunk boundaries, and so
 * the summation order, may differ).
 */
typedef struct tad_paged_kv {
    const int32_t *block_table; /* device int32 [B, max_pages] */
    int32_t max_pages;          /* block-table entries per batch row */
} tad_paged_kv;

int tad_split_paged(const tad_tensor *q, const tad_tensor *k_cache, const tad_tensor *v_cache,
                    const tad_paged_kv *pages, const int32_t *seq_lens, const float *alibi_slopes,
                    int32_t n_splits, void *ws, size_t ws_bytes, hipStream_t stream);

int tad_decode_paged_ws(const tad_tensor *q, const tad_tensor *k_cache, const tad_tensor *v_cache,
                        const tad_paged_kv *pages, const int32_t *seq_lens, const float *alibi_slopes,
                        int32_t n_splits, tad_tensor *out, void *ws, size_t ws_bytes, hipStream_t stream);

int tad_decode_paged(const tad_tensor *q, const tad_tensor *k_cache, const tad_tensor *v_cache,
                     const tad_paged_kv *pages, const int32_t *seq_lens, const float *alibi_slopes,
                     int32_t n_splits, tad_tensor *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TAD_H */
