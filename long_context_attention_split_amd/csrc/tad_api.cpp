// tad_api.cpp -- the C ABI of libtad (declared in include/tad.h): argument
// validation, chunk-count choice, workspace carving and the two kernel launches.
// Every check that can fail runs before anything is launched.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "tad.h"
#include "device_util.h"
#include "tad_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return TAD_OK;
}

int elem_size(int32_t dtype) {
    return dtype == TAD_F32 ? 4 : (dtype == TAD_BF16 ? 2 : 1);
}

bool is_fp8(int32_t dtype) { return dtype == TAD_FP8_E4M3 || dtype == TAD_FP8_E5M2; }

// The kernels' K/V element type for a (validated) tad_dtype.
int kv_type_of(int32_t dtype) {
    return dtype == TAD_F32 ? tad::kKvF32
         : dtype == TAD_BF16 ? tad::kKvBF16
         : dtype == TAD_FP8_E4M3 ? tad::kKvE4M3 : tad::kKvE5M2;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// scale / scale_block of a k or v tensor (dtype already checked).
int check_scales(const tad_tensor *t, const char *name) {
    if (t->scale && !is_fp8(t->dtype))
        return fail(TAD_EINVAL, "%s: a dequantisation scale is only allowed for FP8 tensors", name);
    const int32_t n = t->scale_block;
    if (n == 0) return TAD_OK;
    if (!is_fp8(t->dtype)) return fail(TAD_EINVAL, "%s: scale_block is only allowed for FP8 tensors", name);
    if (!t->scale) return fail(TAD_EINVAL, "%s: scale_block %d without a scale array", name, n);
    if (n < 16 || n > 65536 || (n & (n - 1)))
        return fail(TAD_EUNSUPPORTED, "%s: scale_block must be a power of two from 16 to 65536 (got %d)", name, n);
    return TAD_OK;
}

int log2_of(int32_t n) {
    int lg = 0;
    while ((1 << lg) < n) ++lg;
    return lg;
}

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// Chunk and piece lengths are multiples of this: whole pages, whole K and V scale blocks.
int64_t chunk_align(int64_t page_size, int32_t k_blk, int32_t v_blk) {
    int64_t a = page_size > 1 ? page_size : 1;
    for (int64_t n : {(int64_t)k_blk, (int64_t)v_blk})
        if (n > 1) a = a / gcd64(a, n) * n;
    return a;
}

// Shapes and strides of one decode call, normalised to 4-D [B, H, L, d] views.
struct Problem {
    int64_t B = 0, Hq = 0, Hkv = 0, Lmax = 0, d = 0, nq = 1;
    int32_t q_dtype = 0, kv_dtype = 0;
    int64_t sqb = 0, sqh = 0, sqt = 0;
    int64_t skb = 0, skh = 0, skj = 0;
    int64_t svb = 0, svh = 0, svj = 0;
    const float *k_scale = nullptr, *v_scale = nullptr;
    int32_t k_blk = 0, v_blk = 0;      // keys per scale block (0: one scale per (b, KV head))
    // paged cache (block_table non-null): skh/skj are the head/row strides inside a page
    const int32_t *block_table = nullptr;
    int64_t max_pages = 0, page_size = 0, num_pages = 0, skp = 0, svp = 0;
};

// q or out: [B, H, d] (one token) or [B, H, nq, d].
int parse_query_like(const tad_tensor *t, const char *name, int64_t *B, int64_t *H, int64_t *nq,
                     int64_t *d, int64_t *sb, int64_t *sh, int64_t *st) {
    if (!t) return fail(TAD_EINVAL, "%s: null tensor descriptor", name);
    if (!t->data) return fail(TAD_EINVAL, "%s: null data pointer", name);
    if (t->ndim == 3) {
        *B = t->shape[0]; *H = t->shape[1]; *nq = 1; *d = t->shape[2];
        *sb = t->stride[0]; *sh = t->stride[1]; *st = 0;
        if (t->stride[2] != 1) return fail(TAD_ELAYOUT, "%s: innermost stride must be 1", name);
    } else if (t->ndim == 4) {
        *B = t->shape[0]; *H = t->shape[1]; *nq = t->shape[2]; *d = t->shape[3];
        *sb = t->stride[0]; *sh = t->stride[1]; *st = t->stride[2];
        if (t->stride[3] != 1) return fail(TAD_ELAYOUT, "%s: innermost stride must be 1", name);
    } else {
        return fail(TAD_EINVAL, "%s: ndim must be 3 or 4 (got %d)", name, t->ndim);
    }
    if (*B < 0 || *H < 1 || *d < 1 || *nq < 1) return fail(TAD_EINVAL, "%s: bad shape", name);
    if (*nq > 256) return fail(TAD_EUNSUPPORTED, "%s: at most 256 query tokens per row", name);
    return TAD_OK;
}

// k or v: [B, Hkv, L, d] or [B, L, d].
int parse_kv(const tad_tensor *t, const char *name, int64_t *B, int64_t *H, int64_t *L, int64_t *d,
             int64_t *sb, int64_t *sh, int64_t *sj) {
    if (!t) return fail(TAD_EINVAL, "%s: null tensor descriptor", name);
    if (!t->data) return fail(TAD_EINVAL, "%s: null data pointer", name);
    if (t->ndim == 4) {
        *B = t->shape[0]; *H = t->shape[1]; *L = t->shape[2]; *d = t->shape[3];
        *sb = t->stride[0]; *sh = t->stride[1]; *sj = t->stride[2];
        if (t->stride[3] != 1) return fail(TAD_ELAYOUT, "%s: innermost stride must be 1", name);
    } else if (t->ndim == 3) {
        *B = t->shape[0]; *H = 1; *L = t->shape[1]; *d = t->shape[2];
        *sb = t->stride[0]; *sh = 0; *sj = t->stride[1];
        if (t->stride[2] != 1) return fail(TAD_ELAYOUT, "%s: innermost stride must be 1", name);
    } else {
        return fail(TAD_EINVAL, "%s: ndim must be 3 or 4 (got %d)", name, t->ndim);
    }
    if (*B < 0 || *H < 1 || *L < 0 || *d < 1) return fail(TAD_EINVAL, "%s: bad shape", name);
    if (t->dtype != TAD_F32 && t->dtype != TAD_BF16 && !is_fp8(t->dtype))
        return fail(TAD_EDTYPE, "%s: dtype must be TAD_F32, TAD_BF16, TAD_FP8_E4M3 or TAD_FP8_E5M2", name);
    int rc = check_scales(t, name);
    if (rc) return rc;
    const int64_t es = elem_size(t->dtype);
    if (!aligned16(t->data) || (*sb * es) % 16 || (*sh * es) % 16 || (*sj * es) % 16)
        return fail(TAD_ELAYOUT, "%s: rows must start on 16-byte boundaries", name);
    if (*L > 1 && *sj < *d) return fail(TAD_ELAYOUT, "%s: key stride smaller than d (rows overlap)", name);
    return TAD_OK;
}

int parse_problem(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, Problem *P) {
    int rc;
    int64_t Bq, Hq, dq, nq;
    if ((rc = parse_query_like(q, "q", &Bq, &Hq, &nq, &dq, &P->sqb, &P->sqh, &P->sqt))) return rc;
    if (q->dtype != TAD_F32 && q->dtype != TAD_BF16) return fail(TAD_EDTYPE, "q: dtype must be TAD_F32 or TAD_BF16");
    if (q->scale) return fail(TAD_EINVAL, "q: scale must be NULL");
    const int64_t qes = elem_size(q->dtype);
    if (!aligned16(q->data) || (P->sqb * qes) % 16 || (P->sqh * qes) % 16 || (P->sqt * qes) % 16)
        return fail(TAD_ELAYOUT, "q: rows must start on 16-byte boundaries");
    int64_t Bk, Hk, Lk, dk, Bv, Hv, Lv, dv;
    if ((rc = parse_kv(k, "k", &Bk, &Hk, &Lk, &dk, &P->skb, &P->skh, &P->skj))) return rc;
    if ((rc = parse_kv(v, "v", &Bv, &Hv, &Lv, &dv, &P->svb, &P->svh, &P->svj))) return rc;
    if (k->dtype != v->dtype) return fail(TAD_EDTYPE, "k and v must share a dtype");
    if (Bk != Bv || Hk != Hv || Lk != Lv || dk != dv) return fail(TAD_EINVAL, "k and v shapes differ");
    if (Bk != Bq) return fail(TAD_EINVAL, "batch of q (%lld) and k (%lld) differ", (long long)Bq, (long long)Bk);
    if (dk != dq) return fail(TAD_EINVAL, "head dim of q (%lld) and k (%lld) differ", (long long)dq, (long long)dk);
    if (Hq % Hk) return fail(TAD_EINVAL, "query heads (%lld) not a multiple of KV heads (%lld)", (long long)Hq, (long long)Hk);
    if (dq != 64 && dq != 128 && dq != 256 && dq != 512)
        return fail(TAD_EUNSUPPORTED, "head dim %lld not supported (64, 128, 256, 512)", (long long)dq);
    if (Bq > 0x7fffffff || Hq > 0x7fffffff || Lk > 0x3fffffff)
        return fail(TAD_EUNSUPPORTED, "sizes too large");
    if (Bq * Hq * nq > 0x7fffffff) return fail(TAD_EUNSUPPORTED, "sizes too large");
    P->B = Bq; P->Hq = Hq; P->Hkv = Hk; P->Lmax = Lk; P->d = dq; P->nq = nq;
    P->q_dtype = q->dtype; P->kv_dtype = k->dtype;
    P->k_scale = k->scale; P->v_scale = v->scale;
    P->k_blk = k->scale_block; P->v_blk = v->scale_block;
    return TAD_OK;
}

// k_cache or v_cache of a paged cache: [num_pages, page_size, Hkv, d].
int parse_paged_kv(const tad_tensor *t, const char *name, int64_t *NP, int64_t *PS, int64_t *H, int64_t *d,
                   int64_t *sp, int64_t *sj, int64_t *sh) {
    if (!t) return fail(TAD_EINVAL, "%s: null tensor descriptor", name);
    if (!t->data) return fail(TAD_EINVAL, "%s: null data pointer", name);
    if (t->ndim != 4) return fail(TAD_EINVAL, "%s: a paged cache is 4-D [num_pages, page_size, Hkv, d]", name);
    *NP = t->shape[0]; *PS = t->shape[1]; *H = t->shape[2]; *d = t->shape[3];
    *sp = t->stride[0]; *sj = t->stride[1]; *sh = t->stride[2];
    if (t->stride[3] != 1) return fail(TAD_ELAYOUT, "%s: innermost stride must be 1", name);
    if (*NP < 1 || *PS < 1 || *H < 1 || *d < 1) return fail(TAD_EINVAL, "%s: bad shape", name);
    if (*PS % 16) return fail(TAD_EUNSUPPORTED, "%s: page_size must be a multiple of 16 (got %lld)", name,
                              (long long)*PS);
    if (t->dtype != TAD_BF16 && !is_fp8(t->dtype))
        return fail(TAD_EDTYPE, "%s: a paged cache must be TAD_BF16, TAD_FP8_E4M3 or TAD_FP8_E5M2", name);
    int rc = check_scales(t, name);
    if (rc) return rc;
    const int64_t es = elem_size(t->dtype);
    if (!aligned16(t->data) || (*sp * es) % 16 || (*sj * es) % 16 || (*sh * es) % 16)
        return fail(TAD_ELAYOUT, "%s: rows must start on 16-byte boundaries", name);
    if (*sj < *d) return fail(TAD_ELAYOUT, "%s: row stride smaller than d (rows overlap)", name);
    if (*NP > 0x7fffffff || 16 * *sj * es >= (int64_t(1) << 32))
        return fail(TAD_EUNSUPPORTED, "%s: sizes too large", name);
    return TAD_OK;
}

int parse_paged_problem(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const tad_paged_kv *pages,
                        Problem *P) {
    int rc;
    if (!pages) return fail(TAD_EINVAL, "pages: null descriptor");
    if (!pages->block_table) return fail(TAD_EINVAL, "pages: null block table");
    if (pages->max_pages < 1) return fail(TAD_EINVAL, "pages: max_pages must be >= 1 (got %d)", pages->max_pages);
    int64_t Bq, Hq, dq, nq;
    if ((rc = parse_query_like(q, "q", &Bq, &Hq, &nq, &dq, &P->sqb, &P->sqh, &P->sqt))) return rc;
    if (q->dtype != TAD_F32 && q->dtype != TAD_BF16) return fail(TAD_EDTYPE, "q: dtype must be TAD_F32 or TAD_BF16");
    if (q->scale) return fail(TAD_EINVAL, "q: scale must be NULL");
    const int64_t qes = elem_size(q->dtype);
    if (!aligned16(q->data) || (P->sqb * qes) % 16 || (P->sqh * qes) % 16 || (P->sqt * qes) % 16)
        return fail(TAD_ELAYOUT, "q: rows must start on 16-byte boundaries");
    int64_t NPk, PSk, Hk, dk, NPv, PSv, Hv, dv;
    if ((rc = parse_paged_kv(k, "k_cache", &NPk, &PSk, &Hk, &dk, &P->skp, &P->skj, &P->skh))) return rc;
    if ((rc = parse_paged_kv(v, "v_cache", &NPv, &PSv, &Hv, &dv, &P->svp, &P->svj, &P->svh))) return rc;
    if (k->dtype != v->dtype) return fail(TAD_EDTYPE, "k_cache and v_cache must share a dtype");
    if (NPk != NPv || PSk != PSv || Hk != Hv || dk != dv) return fail(TAD_EINVAL, "k_cache and v_cache shapes differ");
    if (dk != dq) return fail(TAD_EINVAL, "head dim of q (%lld) and k_cache (%lld) differ", (long long)dq, (long long)dk);
    if (Hq % Hk) return fail(TAD_EINVAL, "query heads (%lld) not a multiple of KV heads (%lld)", (long long)Hq, (long long)Hk);
    if (dq != 64 && dq != 128 && dq != 256)
        return fail(TAD_EUNSUPPORTED, "head dim %lld not supported with a paged cache (64, 128, 256)", (long long)dq);
    const int64_t Lmax = (int64_t)pages->max_pages * PSk;
    if (Bq > 0x7fffffff || Hq > 0x7fffffff || Lmax > 0x3fffffff || Bq * Hq * nq > 0x7fffffff)
        return fail(TAD_EUNSUPPORTED, "sizes too large");
    P->B = Bq; P->Hq = Hq; P->Hkv = Hk; P->Lmax = Lmax; P->d = dq; P->nq = nq;
    P->skb = P->svb = 0;
    P->q_dtype = q->dtype; P->kv_dtype = k->dtype;
    P->k_scale = k->scale; P->v_scale = v->scale;
    P->k_blk = k->scale_block; P->v_blk = v->scale_block;
    P->block_table = pages->block_table;
    P->max_pages = pages->max_pages; P->page_size = PSk; P->num_pages = NPk;
    return TAD_OK;
}

int check_out(const tad_tensor *out, const Problem &P, int64_t *sob, int64_t *soh, int64_t *sot) {
    int rc;
    int64_t B, H, d, nq;
    if ((rc = parse_query_like(out, "out", &B, &H, &nq, &d, sob, soh, sot))) return rc;
    if (out->dtype != TAD_F32) return fail(TAD_EDTYPE, "out: dtype must be TAD_F32");
    if (out->scale) return fail(TAD_EINVAL, "out: scale must be NULL");
    if (B != P.B || H != P.Hq || d != P.d || nq != P.nq)
        return fail(TAD_EINVAL, "out: shape must be [B, Hq, (nq,) d] of the inputs");
    return TAD_OK;
}

// 32-bit buffer offsets: one chunk plus a tile of overrun must span < 4 GiB.  And 32-bit
// work counts: no split or pieces kernel launches more than B * Hq * nq * n_splits
// work-groups (the matrix-core kernel B * Hkv * n_splits * column blocks, fewer), which
// the kernels index with 32-bit integers.
int check_offsets(const Problem &P, int64_t S) {
    const int64_t rows = P.B * P.Hq * P.nq;
    if (rows > 0 && S > int64_t(0x7fffffff) / rows)
        return fail(TAD_EUNSUPPORTED, "B * Hq * nq * n_splits = %lld * %lld exceeds 2^31 - 1", (long long)rows,
                    (long long)S);
    const int64_t al = chunk_align(P.block_table ? P.page_size : 1, P.k_blk, P.v_blk);
    if (al > (int64_t(1) << 30))
        return fail(TAD_EUNSUPPORTED, "pages and scale blocks would need chunks of %lld keys", (long long)al);
    if (P.block_table) return TAD_OK;    // paged: one resource per 16-key tile (checked in parse_paged_kv)
    const int64_t es = elem_size(P.kv_dtype);
    const int64_t c = ((P.Lmax + S - 1) / S + al - 1) / al * al;
    const int64_t span_k = (c + 64) * P.skj * es, span_v = (c + 64) * P.svj * es;
    if (span_k >= (int64_t(1) << 32) || span_v >= (int64_t(1) << 32))
        return fail(TAD_EUNSUPPORTED, "chunk spans >= 4 GiB; use more splits");
    return TAD_OK;
}

std::mutex g_cu_mu;
int g_cu_count[64] = {0};

int device_cus(int32_t device, int *cus) {
    int dev = device;
    if (dev < 0) {
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(TAD_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    }
    if (dev >= 64) return fail(TAD_EINVAL, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_cu_mu);
    if (!g_cu_count[dev]) {
        int n = 0;
        hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail(TAD_EHIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
        g_cu_count[dev] = n > 0 ? n : 1;
    }
    *cus = g_cu_count[dev];
    return TAD_OK;
}

// Four (row, KV head, chunk) units per CU; six with several rows, whose lengths may
// differ: then part of the chunks are empty, and the matrix-core kernel, which fits
// the chunk length to the busy ones, gets room to spread a ragged batch over the
// device (grouped-query decode, 8 rows of 4653..26803 keys, FP8 K/V: 58.0 -> 49.9 us
// per step; uniform multi-row batches pay about 1% for the longer merge).  No
// work-group's chunk holds less than 128 KiB of K and V (per KV head: 128 KiB, or
// 32 KiB for grouped-query calls on the matrix-core kernel, which serves them 4 KV heads
// to a work-group when items are many and one KV head otherwise), since shorter
// chunks cost work-group start-up and merge time: 32 bf16 heads of 1024 keys decode
// in 13.5 us with 4 chunks (128 KiB) and 15.4 us with 8; one fp32 d = 512 head of
// 4096 keys in 15.8 us with 128 chunks against ~40 us with the 16 that a fixed
// 256-key minimum gave; 32 query heads over 8 KV heads of 4096 bf16 keys in 15.6 us
// with 64 chunks against 18.0 us with 16.  (tad::kMinChunkBytes = 128 KiB.)
using tad::kMinChunkBytes;

int32_t auto_splits_for(int64_t B, int64_t Hq, int64_t Hkv, int64_t nq, int64_t Lmax, int64_t d,
                        int32_t kv_dtype, int cus) {
    const int64_t units = B * Hkv > 0 ? B * Hkv : 1;
    const int64_t per_cu = B > 1 ? 6 : 4;
    int64_t S = (per_cu * (int64_t)cus + units - 1) / units;
    const int32_t group = (int32_t)(Hq / (Hkv > 0 ? Hkv : 1));
    // mirrors the matrix-core kernel's choice: 4 KV heads per work-group only with one
    // column block per wave (at most 16 (head, token) columns, or d = 256)
    const int64_t heads_per_wg = (Hkv % 4 == 0 && tad::split_mfma_supported((int)d, kv_type_of(kv_dtype), group, (int)nq) &&
                                  ((int64_t)group * nq <= 16 || d == 256)) ? 4 : 1;
    const int64_t by_len = Lmax * 2 * d * elem_size(kv_dtype) * heads_per_wg / kMinChunkBytes;
    if (S > by_len) S = by_len;
    if (S > tad::kMaxSplits) S = tad::kMaxSplits;
    if (S < 1) S = 1;
    return (int32_t)S;
}

// Device arrays of one call: the partials (m, l, o), the arrival counters of the fused
// merge (cnt, one per row), and the pieces' partials (sub_*), which exist when Pmax > 1.
struct WsPtrs {
    float *m, *l, *o;
    int32_t *cnt;
    float *sm, *sl, *so;
    int Pmax;
};

// Pointers into a workspace laid out by tad::ws_layout.  `counters`, when non-null,
// replaces the workspace's own counter region (the no-allocation entry point keeps its
// counters at a fixed place).
void carve_at(char *base, int64_t rows, int64_t S, int64_t d, int32_t *counters, WsPtrs *p) {
    const tad::WsLayout L = tad::ws_layout(rows, S, d);
    p->m = (float *)(base + L.off_m);
    p->l = (float *)(base + L.off_l);
    p->o = (float *)(base + L.off_o);
    p->cnt = counters ? counters : (int32_t *)(base + L.off_cnt);
    p->sm = (float *)(base + L.off_sm);
    p->sl = (float *)(base + L.off_sl);
    p->so = (float *)(base + L.off_so);
    p->Pmax = L.Pmax;
}

int carve_ws(void *ws, size_t ws_bytes, int64_t rows, int64_t S, int64_t d, WsPtrs *p) {
    const tad::WsLayout L = tad::ws_layout(rows, S, d);
    if (!ws) return fail(TAD_EWORKSPACE, "workspace pointer is null");
    if ((uintptr_t)ws & 255u) return fail(TAD_EWORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < L.total)
        return fail(TAD_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
    carve_at((char *)ws, rows, S, d, nullptr, p);
    return TAD_OK;
}

// Pieces per chunk (SplitArgs::P) for a call the vector kernel serves with one query
// row per KV head: up to the workspace's Pmax (which brings the (row, chunk) pairs to
// about kSubSplitTarget work-groups), and no piece under kMinChunkBytes of K and V, the
// shortest chunk the automatic count gives.  A function of the call's sizes only, so
// tad_split and the decode entry points cut a call the same way.
int pieces_for(const Problem &P, int32_t S, int Pmax) {
    if (Pmax <= 1) return 1;
    const int64_t c = (P.Lmax + S - 1) / S;
    const int64_t n = c * 2 * P.d * elem_size(P.kv_dtype) / kMinChunkBytes;
    return (int)(n < 1 ? 1 : (n > Pmax ? Pmax : n));
}

// Output of a decode: fp32 [B, Hq, nq, d] with element strides.
struct OutDesc {
    float *data = nullptr;
    int64_t sob = 0, soh = 0, sot = 0;
};

// Kernel arguments of a split launch.  With out.data non-null the kernel also merges
// (fused: the last work-group of each row merges it, using the workspace's arrival
// counters).
tad::SplitArgs split_args(const Problem &P, const tad_tensor *q, const tad_tensor *k, const tad_tensor *v,
                          const int32_t *seq_lens, const float *slopes, int32_t S, const WsPtrs &w,
                          const OutDesc &out) {
    tad::SplitArgs a;
    a.q = q->data; a.sqb = P.sqb; a.sqh = P.sqh; a.sqt = P.sqt; a.q_bf16 = P.q_dtype == TAD_BF16;
    a.nq = (int32_t)P.nq;
    a.k = k->data; a.v = v->data;
    a.kv_type = kv_type_of(P.kv_dtype);
    a.k_scale = P.k_scale; a.v_scale = P.v_scale;
    a.k_blk_lg = P.k_blk ? log2_of(P.k_blk) : 0;
    a.v_blk_lg = P.v_blk ? log2_of(P.v_blk) : 0;
    a.k_nblk = P.k_blk ? (int32_t)((P.Lmax + P.k_blk - 1) / P.k_blk) : 0;
    a.v_nblk = P.v_blk ? (int32_t)((P.Lmax + P.v_blk - 1) / P.v_blk) : 0;
    a.align = (int32_t)chunk_align(P.block_table ? P.page_size : 1, P.k_blk, P.v_blk);
    a.skb = P.skb; a.skh = P.skh; a.skj = P.skj;
    a.svb = P.svb; a.svh = P.svh; a.svj = P.svj;
    a.seq_lens = seq_lens; a.slopes = slopes;
    a.block_table = P.block_table;
    a.max_pages = (int32_t)P.max_pages; a.page_size = (int32_t)P.page_size; a.num_pages = (int32_t)P.num_pages;
    a.skp = P.skp; a.svp = P.svp;
    a.B = (int32_t)P.B; a.Hq = (int32_t)P.Hq; a.Hkv = (int32_t)P.Hkv; a.Lmax = (int32_t)P.Lmax;
    a.S = S; a.group = (int32_t)(P.Hq / P.Hkv);
    int cus = 0;
    a.cus = device_cus(-1, &cus) == TAD_OK ? cus : 0;     // 0: the chunk-length fit is skipped
    a.wg_slots = 0;
    a.qscale = (float)(1.4426950408889634 / sqrt((double)P.d));
    a.ws_m = w.m; a.ws_l = w.l; a.ws_o = w.o;
    a.fused = 0;
    a.cnt = w.cnt;
    a.out = out.data;
    a.sob = out.sob; a.soh = out.soh; a.sot = out.sot;
    a.P = 1;
    a.sub_m = w.sm; a.sub_l = w.sl; a.sub_o = w.so;
    // pieces: only where the vector kernel runs with one query row per KV head
    if (a.group * a.nq == 1 && !tad::split_mfma_supported((int)P.d, a.kv_type, a.group, a.nq) &&
        !tad::split_heads_supported(a, (int)P.d))
        a.P = pieces_for(P, S, w.Pmax);
    a.fused = out.data != nullptr;
    return a;
}

// Launch the split kernel.  Kernel choice: query-head groups and several tokens on the
// matrix cores; caches whose heads are interleaved per key (one query head per KV
// head) on the head-packed vector kernel; everything else on the vector kernel.  Chunks read as pieces (a.P > 1) are then pre-merged by pieces_kernel, so the
// workspace holds the chunk partials when the launches are done; with merge_out the
// pieces kernel also merges each row into merge_out (its last work-group per row).
int launch_split(const tad::SplitArgs &a, int64_t d, hipStream_t stream, const OutDesc *merge_out = nullptr) {
    hipError_t e;
    if (tad::split_mfma_supported((int)d, a.kv_type, a.group, a.nq))
        e = tad::launch_split_mfma(a, (int)d, stream);
    else if (tad::split_heads_supported(a, (int)d))
        e = tad::launch_split_heads(a, (int)d, stream);
    else
        e = tad::launch_split_valu(a, (int)d, stream);
    if (e != hipSuccess) return fail(TAD_EHIP, "split kernel launch: %s", hipGetErrorString(e));
    if (a.P > 1) {
        tad::PiecesArgs pa;
        pa.sub_m = a.sub_m; pa.sub_l = a.sub_l; pa.sub_o = a.sub_o;
        pa.ws_m = a.ws_m; pa.ws_l = a.ws_l; pa.ws_o = a.ws_o;
        pa.chunks = (int64_t)a.B * a.Hq * a.nq * a.S;
        pa.P = a.P;
        pa.S = a.S; pa.Hq = a.Hq;
        pa.cnt = a.cnt;
        pa.out = merge_out ? merge_out->data : nullptr;
        pa.sob = merge_out ? merge_out->sob : 0;
        pa.soh = merge_out ? merge_out->soh : 0;
        e = tad::launch_pieces(pa, (int)d, stream);
        if (e != hipSuccess) return fail(TAD_EHIP, "pieces kernel launch: %s", hipGetErrorString(e));
    }
    return TAD_OK;
}

int launch_merge(int64_t B, int64_t Hq, int64_t nq, int32_t S, int64_t d, const WsPtrs &w, const OutDesc &out,
                 hipStream_t stream) {
    tad::CombineArgs c;
    c.ws_m = w.m; c.ws_l = w.l; c.ws_o = w.o;
    c.out = out.data; c.sob = out.sob; c.soh = out.soh; c.sot = out.sot;
    c.B = (int32_t)B; c.Hq = (int32_t)Hq; c.nq = (int32_t)nq; c.S = S;
    hipError_t e = tad::launch_combine(c, (int)d, stream);
    if (e != hipSuccess) return fail(TAD_EHIP, "combine kernel launch: %s", hipGetErrorString(e));
    return TAD_OK;
}

int check_splits(int32_t S) {
    if (S < 1 || S > tad::kMaxSplits)
        return fail(TAD_EINVAL, "n_splits must be in [1, %d] (got %d)", tad::kMaxSplits, S);
    return TAD_OK;
}

// Split + merge.  Small grids (at most 8 chunks, fewer (row, chunk) pairs than compute
// units) are launch-bound, and there one launch with the merge fused into the split
// kernel wins when the call is launched eagerly: the vector kernel's last work-group
// per row merges the row (13.6 vs 15.5 us for 32 heads x 1024 keys), the matrix-core
// kernel's last work-group per (row, KV head) merges that KV head's rows side by side
// (one row of 32 query heads over 8 KV heads, 4096 keys at 8 chunks: 15.6 vs 18.4 us
// per call through the Python binding; in a replayed graph 13.3 vs 13.0-13.2 us), and
// the head-packed kernel's last work-group per (row, 4-head group) merges those 4
// rows; a call whose chunks are read as pieces takes two launches, the pieces kernel's
// last work-group per row merging it.  With more chunks one work-group's merge costs
// more than the combine kernel (graph replay, the grouped-query call at 32 chunks: 13.1
// vs 9.9 us), so larger grids run split and combine.  Both forms give bit-identical
// outputs (the merges keep the combine's summation order).
int run_decode(const Problem &P, const tad_tensor *q, const tad_tensor *k, const tad_tensor *v,
               const int32_t *seq_lens, const float *slopes, int32_t S, const WsPtrs &w,
               const OutDesc &out, hipStream_t stream) {
    int cus = 0;
    int rc = device_cus(-1, &cus);
    if (rc) return rc;
    const tad::SplitArgs unfused = split_args(P, q, k, v, seq_lens, slopes, S, w, OutDesc());
    const bool mfma = tad::split_mfma_supported((int)P.d, unfused.kv_type, unfused.group, unfused.nq);
    const bool heads = !mfma && tad::split_heads_supported(unfused, (int)P.d);
    const bool vector_kernel = !mfma && !heads;
    const bool small = S <= tad::kMaxFusedSplits;
    if ((vector_kernel && unfused.P == 1 && small && P.B * P.Hq * P.nq * (int64_t)S < cus) ||
        (mfma && small && P.B * P.Hkv * (int64_t)S <= cus && tad::split_mfma_fusable(unfused, (int)P.d)) ||
        (heads && small && P.B * (P.Hq / 4) * (int64_t)S <= cus))
        return launch_split(split_args(P, q, k, v, seq_lens, slopes, S, w, out), P.d, stream);
    // chunks read as pieces: the pieces kernel's last work-group per row merges it
    if (vector_kernel && unfused.P > 1 && small && P.B * P.Hq * P.nq * (int64_t)S <= cus)
        return launch_split(unfused, P.d, stream, &out);
    if ((rc = launch_split(unfused, P.d, stream))) return rc;
    return launch_merge(P.B, P.Hq, P.nq, S, P.d, w, out, stream);
}

// Validation shared by the decode entry points (pages non-null: paged cache);
// resolves automatic n_splits.
int prepare_decode(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const tad_paged_kv *pages,
                   int32_t n_splits, const tad_tensor *out, Problem *P, int32_t *S, OutDesc *od) {
    int rc;
    if ((rc = pages ? parse_paged_problem(q, k, v, pages, P) : parse_problem(q, k, v, P))) return rc;
    if ((rc = check_out(out, *P, &od->sob, &od->soh, &od->sot))) return rc;
    od->data = (float *)out->data;
    if (n_splits <= 0) {
        int cus = 0;
        if ((rc = device_cus(-1, &cus))) return rc;
        *S = auto_splits_for(P->B, P->Hq, P->Hkv, P->nq, P->Lmax, P->d, P->kv_dtype, cus);
    } else {
        *S = n_splits;
    }
    if ((rc = check_splits(*S))) return rc;
    return check_offsets(*P, *S);
}

int split_impl(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const tad_paged_kv *pages,
               const int32_t *seq_lens, const float *alibi_slopes, int32_t n_splits, void *ws, size_t ws_bytes,
               hipStream_t stream) {
    Problem P;
    int rc;
    if ((rc = pages ? parse_paged_problem(q, k, v, pages, &P) : parse_problem(q, k, v, &P))) return rc;
    if ((rc = check_splits(n_splits))) return rc;
    if ((rc = check_offsets(P, n_splits))) return rc;
    WsPtrs w;
    if ((rc = carve_ws(ws, ws_bytes, P.B * P.Hq * P.nq, n_splits, P.d, &w))) return rc;
    if (P.B == 0) return ok();
    if ((rc = launch_split(split_args(P, q, k, v, seq_lens, alibi_slopes, n_splits, w, OutDesc()), P.d, stream)))
        return rc;
    return ok();
}

int decode_ws_impl(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const tad_paged_kv *pages,
                   const int32_t *seq_lens, const float *alibi_slopes, int32_t n_splits, tad_tensor *out, void *ws,
                   size_t ws_bytes, hipStream_t stream) {
    Problem P;
    int32_t S;
    OutDesc od;
    int rc;
    if ((rc = prepare_decode(q, k, v, pages, n_splits, out, &P, &S, &od))) return rc;
    WsPtrs w;
    if ((rc = carve_ws(ws, ws_bytes, P.B * P.Hq * P.nq, S, P.d, &w))) return rc;
    if (P.B == 0) return ok();
    if ((rc = run_decode(P, q, k, v, seq_lens, alibi_slopes, S, w, od, stream))) return rc;
    return ok();
}

int decode_impl(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const tad_paged_kv *pages,
                const int32_t *seq_lens, const float *alibi_slopes, int32_t n_splits, tad_tensor *out,
                hipStream_t stream) {
    Problem P;
    int32_t S;
    OutDesc od;
    int rc;
    if ((rc = prepare_decode(q, k, v, pages, n_splits, out, &P, &S, &od))) return rc;
    if (P.B == 0) return ok();
    const int64_t rows = P.B * P.Hq * P.nq;
    const size_t bytes = tad::ws_layout(rows, S, P.d).total;
    void *ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, bytes, stream);
    if (e != hipSuccess) return fail(TAD_EHIP, "hipMallocAsync(%zu): %s", bytes, hipGetErrorString(e));
    WsPtrs w;
    rc = carve_ws(ws, bytes, rows, S, P.d, &w);
    if (!rc) {
        hipError_t ez = tad::launch_fill_zero(w.cnt, tad::ws_counters(rows, S, P.d), stream);
        if (ez != hipSuccess) rc = fail(TAD_EHIP, "counter clear launch: %s", hipGetErrorString(ez));
    }
    if (!rc) rc = run_decode(P, q, k, v, seq_lens, alibi_slopes, S, w, od, stream);
    e = hipFreeAsync(ws, stream);
    if (rc) return rc;
    if (e != hipSuccess) return fail(TAD_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
    return ok();
}

// ---- Scratch of tad_decode_noalloc: a file-scope device array, one copy per device
// (HIP places a module's __device__ variables on every device that loads it; each
// copy lives until the process ends).  Its first kScratchCounterBytes hold the arrival
// counters, which must start at zero: they are cleared once per device, and every
// call that completes leaves them zero.  The rest holds one call's partials, laid out
// as a workspace (tad::ws_layout).  In host code `scratch` names a host-side stand-in,
// not the device memory: only the address hipGetSymbolAddress returns for the current
// device is ever passed on.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr size_t kScratchCounterBytes = size_t(256) << 10;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
char *g_scratch_ptr[64] = {nullptr};
bool g_scratch_zeroed[64] = {false};

// The current device's copy of `scratch` (looked up once per device), with its counters
// cleared by a kernel on `stream` the first time.  A clear recorded into a stream that
// is being captured only runs when the graph does, so it is repeated until one is
// issued outside a capture.
int scratch_of_device(hipStream_t stream, char **base) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TAD_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(TAD_EINVAL, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(TAD_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = (char *)p;
    }
    if (!g_scratch_zeroed[dev]) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return fail(TAD_EHIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
        e = tad::launch_fill_zero((int32_t *)g_scratch_ptr[dev], (int64_t)(kScratchCounterBytes / 4), stream);
        if (e != hipSuccess) return fail(TAD_EHIP, "scratch counter clear launch: %s", hipGetErrorString(e));
        if (cs == hipStreamCaptureStatusNone) g_scratch_zeroed[dev] = true;
    }
    *base = g_scratch_ptr[dev];
    return TAD_OK;
}

int decode_noalloc_impl(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const int32_t *seq_lens,
                        const float *alibi_slopes, int32_t n_splits, tad_tensor *out, hipStream_t stream) {
    Problem P;
    int32_t S;
    OutDesc od;
    int rc;
    if ((rc = prepare_decode(q, k, v, nullptr, n_splits, out, &P, &S, &od))) return rc;
    const int64_t rows = P.B * P.Hq * P.nq;
    const size_t need = tad::ws_layout(rows, S, P.d).total;
    const int64_t counters = tad::ws_counters(rows, S, P.d);
    if (need > kScratchBytes - kScratchCounterBytes || counters > (int64_t)(kScratchCounterBytes / 4))
        return fail(TAD_EWORKSPACE,
                    "tad_decode_noalloc: this call needs %zu bytes of partials and %lld counters; the scratch "
                    "holds %zu bytes and %zu counters (use tad_decode_ws with a workspace)",
                    need, (long long)counters, kScratchBytes - kScratchCounterBytes, kScratchCounterBytes / 4);
    if (P.B == 0) return ok();
    char *base = nullptr;
    if ((rc = scratch_of_device(stream, &base))) return rc;
    WsPtrs w;
    carve_at(base + kScratchCounterBytes, rows, S, P.d, (int32_t *)base, &w);
    if ((rc = run_decode(P, q, k, v, seq_lens, alibi_slopes, S, w, od, stream))) return rc;
    return ok();
}

}  // namespace

extern "C" {

int tad_version(void) { return TAD_VERSION; }

const char *tad_last_error(void) { return g_last_error.c_str(); }

int32_t tad_auto_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t nq, int64_t Lmax, int32_t d, int32_t kv_dtype,
                        int32_t device) {
    if (B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || nq < 1 || nq > 256 || Lmax < 0)
        return fail(TAD_EINVAL, "tad_auto_splits: bad sizes");
    if (d != 64 && d != 128 && d != 256 && d != 512) return fail(TAD_EUNSUPPORTED, "tad_auto_splits: d = %d", d);
    if (kv_dtype != TAD_F32 && kv_dtype != TAD_BF16 && !is_fp8(kv_dtype))
        return fail(TAD_EDTYPE, "tad_auto_splits: K/V dtype %d", kv_dtype);
    int cus = 0;
    int rc = device_cus(device, &cus);
    if (rc) return rc;
    ok();
    return auto_splits_for(B, Hq, Hkv, nq, Lmax, d, kv_dtype, cus);
}

size_t tad_workspace_bytes(int32_t B, int32_t Hq, int32_t nq, int32_t n_splits, int32_t d) {
    if (B < 1 || Hq < 1 || nq < 1 || n_splits < 1 || d < 1) return 0;
    return tad::ws_layout((int64_t)B * Hq * nq, n_splits, d).total;
}

int tad_workspace_clear(void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!ws) return fail(TAD_EWORKSPACE, "workspace pointer is null");
    if ((uintptr_t)ws & 255u) return fail(TAD_EWORKSPACE, "workspace must be 256-byte aligned");
    hipError_t e = tad::launch_fill_zero((int32_t *)ws, (int64_t)(ws_bytes / sizeof(int32_t)), stream);
    if (e != hipSuccess) return fail(TAD_EHIP, "workspace clear launch: %s", hipGetErrorString(e));
    return ok();
}

int tad_split(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const int32_t *seq_lens,
              const float *alibi_slopes, int32_t n_splits, void *ws, size_t ws_bytes, hipStream_t stream) {
    return split_impl(q, k, v, nullptr, seq_lens, alibi_slopes, n_splits, ws, ws_bytes, stream);
}

int tad_split_paged(const tad_tensor *q, const tad_tensor *k_cache, const tad_tensor *v_cache,
                    const tad_paged_kv *pages, const int32_t *seq_lens, const float *alibi_slopes,
                    int32_t n_splits, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!pages) return fail(TAD_EINVAL, "pages: null descriptor");
    return split_impl(q, k_cache, v_cache, pages, seq_lens, alibi_slopes, n_splits, ws, ws_bytes, stream);
}

int tad_combine(const void *ws, size_t ws_bytes, int32_t B, int32_t Hq, int32_t nq, int32_t n_splits,
                int32_t d, tad_tensor *out, hipStream_t stream) {
    int rc;
    if (B < 0 || Hq < 1 || nq < 1) return fail(TAD_EINVAL, "tad_combine: bad B, Hq or nq");
    if (d != 64 && d != 128 && d != 256 && d != 512)
        return fail(TAD_EUNSUPPORTED, "head dim %d not supported (64, 128, 256, 512)", d);
    if ((rc = check_splits(n_splits))) return rc;
    Problem P;
    P.B = B; P.Hq = Hq; P.d = d; P.nq = nq;
    OutDesc od;
    if ((rc = check_out(out, P, &od.sob, &od.soh, &od.sot))) return rc;
    od.data = (float *)out->data;
    WsPtrs w;
    if ((rc = carve_ws(const_cast<void *>(ws), ws_bytes, (int64_t)B * Hq * nq, n_splits, d, &w))) return rc;
    if (B == 0) return ok();
    if ((rc = launch_merge(B, Hq, nq, n_splits, d, w, od, stream))) return rc;
    return ok();
}

int tad_decode_ws(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const int32_t *seq_lens,
                  const float *alibi_slopes, int32_t n_splits, tad_tensor *out, void *ws, size_t ws_bytes,
                  hipStream_t stream) {
    return decode_ws_impl(q, k, v, nullptr, seq_lens, alibi_slopes, n_splits, out, ws, ws_bytes, stream);
}

int tad_decode(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const int32_t *seq_lens,
               const float *alibi_slopes, int32_t n_splits, tad_tensor *out, hipStream_t stream) {
    return decode_impl(q, k, v, nullptr, seq_lens, alibi_slopes, n_splits, out, stream);
}

int tad_decode_noalloc(const tad_tensor *q, const tad_tensor *k, const tad_tensor *v, const int32_t *seq_lens,
                       const float *alibi_slopes, int32_t n_splits, tad_tensor *out, hipStream_t stream) {
    return decode_noalloc_impl(q, k, v, seq_lens, alibi_slopes, n_splits, out, stream);
}

int tad_decode_paged_ws(const tad_tensor *q, const tad_tensor *k_cache, const tad_tensor *v_cache,
                        const tad_paged_kv *pages, const int32_t *seq_lens, const float *alibi_slopes,
                        int32_t n_splits, tad_tensor *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!pages) return fail(TAD_EINVAL, "pages: null descriptor");
    return decode_ws_impl(q, k_cache, v_cache, pages, seq_lens, alibi_slopes, n_splits, out, ws, ws_bytes, stream);
}

int tad_decode_paged(const tad_tensor *q, const tad_tensor *k_cache, const tad_tensor *v_cache,
                     const tad_paged_kv *pages, const int32_t *seq_lens, const float *alibi_slopes,
                     int32_t n_splits, tad_tensor *out, hipStream_t stream) {
    if (!pages) return fail(TAD_EINVAL, "pages: null descriptor");
    return decode_impl(q, k_cache, v_cache, pages, seq_lens, alibi_slopes, n_splits, out, stream);
}

}  // extern "C"
