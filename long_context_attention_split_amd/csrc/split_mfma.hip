// split_mfma.hip -- split step for grouped-query attention on the matrix cores (gfx950).
//
// With g query heads sharing one KV head, the scores of a key tile form a real
// dense product S^T[key][head] = K_tile . Q^T, and so does the value update
// O^T[e][head] += V_tile^T . P^T.  One work-group (4 waves) owns one (b, kv head,
// chunk) and all g query heads of the group, so every K and V byte of the chunk is
// read from HBM once (with the non-temporal policy) however many heads share it.
// The per-head partials (m, l, o) it writes are the same as the vector-ALU kernel's
// (see split_valu.hip): chunk maximum in base 2, sum of 2^(s - m), and the
// 2^(s - m)-weighted sum of value rows, i.e. the per-chunk local max, denominator
// and numerator of tree_attn_decode ("Tree Attention Decoding").
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Lane l holds A[i][k] for i = l%16 and
// B[k][j] for j = l%16, with k in the 8-wide block l/16, and C[i][j] for
// j = l%16, i = 4*(l/16) + r, r = 0..3.  The reduction index only has to be laid out
// the same way in A and B, which the code below does by construction.
//
//  * scores: A = 16 keys x 32 dims of K (lane: key l%16, dims 32kk + 8(l/16) .. +7,
//    one 16-byte load), B = Q^T with heads on the 16 columns (zero past g).  fp32 q
//    is split into bf16 hi + lo and both are multiplied (two MFMAs), which keeps the
//    scores at ~16 significant bits of q; K is exactly bf16.  Result: lane l holds
//    the scores of keys 4(l/16)+r of the subtile for head l%16.
//  * transpose: multiplying the same K-style A operand of V by a 0/1 selector
//    B[k][j] = (k == j + 16h) gives C[key][j] = V[key][32kk + 16h + j]: lane l then
//    holds 4 keys of one value column -- the transposed layout the value product
//    needs.  The values are exact bf16 and the product is exact.
//  * value update: A = V^T (16 value columns x 32 keys: the 4 keys of each of two
//    subtiles), B = P^T (32 keys x heads), with the probabilities split into bf16
//    hi + lo (two MFMAs, ~16-bit weights).  The key order inside the 32-wide
//    reduction is the same permutation on both sides, so it needs no shuffle.
//
// Softmax per head: lane l owns head l%16 and 8 of the tile's 32 keys; the four
// lanes l, l^16, l^32, l^48 together hold the tile and exchange their max and sum.
// The running (m, l) and the rescale of O by 2^(m_old - m_new) follow the online
// softmax of the "Flash Aandacht" page's block loop, kept un-normalised.

#include "device_util.h"
#include "tad_internal.h"

namespace tad {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two fp32 values that are exact bf16 numbers -> one packed dword (x in the low half).
__device__ __forceinline__ uint32_t pack_exact_bf16(float x, float y) {
    return (__float_as_uint(x) >> 16) | (__float_as_uint(y) & 0xffff0000u);
}

// x = hi + lo with hi, lo bf16 (truncations): |x - hi - lo| <= 2^-16 |x|.
__device__ __forceinline__ void split_bf16(float x, uint32_t &hi, uint32_t &lo) {
    const uint32_t h = __float_as_uint(x) & 0xffff0000u;
    const float r = x - __uint_as_float(h);              // exact
    hi = h >> 16;
    lo = __float_as_uint(r) >> 16;
}

template <int D>
__global__ __launch_bounds__(kSplitThreads) void split_mfma_kernel(SplitArgs a) {
    static_assert(D == 64 || D == 128, "head dim");
    constexpr int NKK = D / 32;          // 32-wide slices of d (score reduction)
    constexpr int NB = D / 16;           // 16-wide column blocks of the output
    constexpr int TK = 32;               // keys per wave tile (two 16-key subtiles)
    constexpr int NW = kSplitThreads / 64;
    constexpr int MAXG = 16;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c4 = lane >> 4;            // 8-wide reduction block of this lane
    const int j16 = lane & 15;           // column (head) / row (key, value column)

    const int S = a.S, g = a.group;
    const int s = blockIdx.x % S;
    const int bk = blockIdx.x / S;
    const int b = bk / a.Hkv, kvh = bk % a.Hkv;
    const bool head_ok = j16 < g;
    const int h = kvh * g + (head_ok ? j16 : 0);

    int L = a.Lmax;
    if (a.seq_lens) L = min(max(a.seq_lens[b], 0), a.Lmax);
    const int c = (L + S - 1) / S;
    const int j0 = (int)min((int64_t)s * c, (int64_t)L);
    const int j1 = min(j0 + c, L);
    const int n = j1 - j0;

    const uint32_t krow = (uint32_t)(a.skj * 2), vrow = (uint32_t)(a.svj * 2);
    const char *kbase = (const char *)a.k + ((int64_t)b * a.skb + (int64_t)kvh * a.skh + (int64_t)j0 * a.skj) * 2;
    const char *vbase = (const char *)a.v + ((int64_t)b * a.svb + (int64_t)kvh * a.svh + (int64_t)j0 * a.svj) * 2;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase, (uint32_t)n * krow);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase, (uint32_t)n * vrow);

    // ---- B operands of the score product: q of head j16, dims 32kk + 8c4 + t, as hi/lo.
    uint4 qhi[NKK], qlo[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        float x[8];
        const int64_t qoff = (int64_t)b * a.sqb + (int64_t)h * a.sqh + 32 * kk + 8 * c4;
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
        for (int t = 0; t < 8; ++t) split_bf16(head_ok ? x[t] * a.qscale : 0.f, hw[t], lw[t]);
        qhi[kk] = make_uint4(hw[0] | hw[1] << 16, hw[2] | hw[3] << 16, hw[4] | hw[5] << 16, hw[6] | hw[7] << 16);
        qlo[kk] = make_uint4(lw[0] | lw[1] << 16, lw[2] | lw[3] << 16, lw[4] | lw[5] << 16, lw[6] | lw[7] << 16);
    }
    // ---- selector B operands for the transpose: element t is 1 where 8*c4 + t == j16 + 16*half.
    uint4 sel[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t0 = 8 * c4 + 2 * i - 16 * half;
            const uint32_t lo16 = (t0 == j16) ? 0x3F80u : 0u;       // bf16 1.0
            const uint32_t hi16 = (t0 + 1 == j16) ? 0x3F80u : 0u;
            w[i] = lo16 | (hi16 << 16);
        }
        sel[half] = make_uint4(w[0], w[1], w[2], w[3]);
    }

    const float slope2 = (a.slopes && head_ok) ? a.slopes[h] * 1.4426950408889634f : 0.f;
    const bool alibi = a.slopes != nullptr;

    float m = kNegInf, l = 0.f;
    f32x4_t O[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) O[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

    for (int t0 = wave * TK; t0 < n; t0 += NW * TK) {
        uint4 kraw[2][NKK], vraw[2][NKK];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                kraw[sub][kk] = load16<kPolicyNT>(kr, (uint32_t)(t0 + 16 * sub + j16) * krow + 64u * kk + 16u * c4);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                vraw[sub][kk] = load16<kPolicyNT>(vr, (uint32_t)(t0 + 16 * sub + j16) * vrow + 64u * kk + 16u * c4);

        // scores: sc[sub][r] is key t0 + 16 sub + 4 c4 + r, head j16
        f32x4_t sc[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            f32x4_t acc = zero4;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                acc = mfma16x16x32(kraw[sub][kk], qhi[kk], acc);
                acc = mfma16x16x32(kraw[sub][kk], qlo[kk], acc);
            }
            sc[sub] = acc;
        }
        float p[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int key = t0 + 16 * (t >> 2) + 4 * c4 + (t & 3);
            float x = sc[t >> 2][t & 3];
            if (alibi) x = fmaf(slope2, (float)(j0 + key - (L - 1)), x);
            p[t] = (key < n) ? x : kNegInf;
        }
        float mt = p[0];
#pragma unroll
        for (int t = 1; t < 8; ++t) mt = fmaxf(mt, p[t]);
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m, mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2_fast(m - m_use);
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            p[t] = exp2_fast(p[t] - m_use);
            ps += p[t];
        }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l = fmaf(l, alpha, ps);
        m = m_new;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nb] *= alpha;

        // P^T operands: reduction slot t of this lane is key t0 + 16 (t>>2) + 4 c4 + (t&3)
        uint32_t ph[8], pl[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) split_bf16(p[t], ph[t], pl[t]);
        const uint4 phi = make_uint4(ph[0] | ph[1] << 16, ph[2] | ph[3] << 16, ph[4] | ph[5] << 16, ph[6] | ph[7] << 16);
        const uint4 plo = make_uint4(pl[0] | pl[1] << 16, pl[2] | pl[3] << 16, pl[4] | pl[5] << 16, pl[6] | pl[7] << 16);

        // V^T blocks (same key slots), then the value update
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const f32x4_t v0 = mfma16x16x32(vraw[0][kk], sel[half], zero4);
                const f32x4_t v1 = mfma16x16x32(vraw[1][kk], sel[half], zero4);
                const uint4 vt = make_uint4(pack_exact_bf16(v0[0], v0[1]), pack_exact_bf16(v0[2], v0[3]),
                                            pack_exact_bf16(v1[0], v1[1]), pack_exact_bf16(v1[2], v1[3]));
                const int nb = 2 * kk + half;
                O[nb] = mfma16x16x32(vt, phi, O[nb]);
                O[nb] = mfma16x16x32(vt, plo, O[nb]);
            }
        }
    }

    // ---- merge the NW wave states per head through LDS, then write the partials.
    __shared__ float lds_o[NW][MAXG][D];
    __shared__ float lds_m[NW][MAXG], lds_l[NW][MAXG];
    if (head_ok) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) lds_o[wave][j16][16 * nb + 4 * c4 + r] = O[nb][r];
        if (c4 == 0) {
            lds_m[wave][j16] = m;
            lds_l[wave][j16] = l;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < g * D; idx += kSplitThreads) {
        const int hh = idx / D, e = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_m[w][hh]);
        const float Mu = (M == kNegInf) ? 0.f : M;
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float sw = exp2_fast(lds_m[w][hh] - Mu);
            acc = fmaf(sw, lds_o[w][hh][e], acc);
            lsum = fmaf(sw, lds_l[w][hh], lsum);
        }
        const int64_t r = ((int64_t)b * a.Hq + kvh * g + hh) * S + s;
        a.ws_o[r * D + e] = acc;
        if (e == 0) {
            a.ws_m[r] = M;
            a.ws_l[r] = lsum;
        }
    }
}

bool split_mfma_supported(int d, bool kv_bf16, int group) {
    return kv_bf16 && group >= 2 && group <= 16 && (d == 64 || d == 128);
}

hipError_t launch_split_mfma(const SplitArgs &a, int d, hipStream_t st) {
    const int64_t grid = (int64_t)a.B * a.Hkv * a.S;
    if (grid <= 0) return hipSuccess;
    switch (d) {
        case 64: hipLaunchKernelGGL(split_mfma_kernel<64>, dim3((unsigned)grid), dim3(kSplitThreads), 0, st, a); break;
        case 128: hipLaunchKernelGGL(split_mfma_kernel<128>, dim3((unsigned)grid), dim3(kSplitThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tad
