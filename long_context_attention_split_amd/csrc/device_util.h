// device_util.h -- small gfx950 building blocks used by the decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tad {

constexpr float kNegInf = -__builtin_inff();

// Buffer resource over [base, base + bytes): loads past `bytes` return zero, which is
// how chunk tails and ragged sequence ends are kept from reading out of range.
// Word 3 = 0x00020000 is the raw (untyped, 32-bit data format) setting for gfx9 parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Cache-policy bits of a gfx950 buffer load: NT marks the data as streaming
// (read once), which keeps a long K/V sweep from churning L2 and the memory-side
// cache; on MI355X it lifts a pure read stream from ~6.2 to ~7.1 TB/s.
constexpr int kPolicyDefault = 0;
constexpr int kPolicyNT = 2;

// 16-byte load through a buffer resource; `off` is a byte offset from the base.
template <int POLICY = kPolicyDefault>
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY));
}

// bf16 pair in one dword -> two fp32 (bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element types of K and V (values of SplitArgs::kv_type).
constexpr int kKvF32 = 0, kKvBF16 = 1, kKvE4M3 = 2, kKvE5M2 = 3;

// The slice of one key row a lane holds: EPL consecutive elements, loaded with one
// 16-byte load (bf16: 8 elements, FP8: 16) or two (fp32: 8), then widened to fp32.
// FP8 uses the hardware OCP E4M3 / E5M2 conversions (v_cvt_pk_f32_fp8 / _bf8, two
// elements per instruction; exact).
template <int KVT, int POLICY>
struct RowChunk {
    static constexpr int kLoads = KVT == kKvF32 ? 2 : 1;
    static constexpr int EPL = (KVT == kKvE4M3 || KVT == kKvE5M2) ? 16 : 8;
    static constexpr int kBytes = 16 * kLoads;        // bytes per lane per key
    uint4 raw[kLoads];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) raw[i] = load16<POLICY>(r, off + 16u * i);
    }
    __device__ __forceinline__ void widen(float (&f)[EPL]) const {
        if constexpr (KVT == kKvF32) {
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = __uint_as_float((&raw[e >> 2].x)[e & 3]);
        } else if constexpr (KVT == kKvBF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = (&raw[0].x)[i];
                f[2 * i] = bf16_lo(w);
                f[2 * i + 1] = bf16_hi(w);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int w = (int)(&raw[0].x)[i];
                typedef float f2_t __attribute__((ext_vector_type(2)));
                f2_t lo, hi;
                if constexpr (KVT == kKvE4M3) {
                    lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
                    hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
                } else {
                    lo = __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
                    hi = __builtin_amdgcn_cvt_pk_f32_bf8(w, true);
                }
                f[4 * i] = lo.x; f[4 * i + 1] = lo.y; f[4 * i + 2] = hi.x; f[4 * i + 3] = hi.y;
            }
        }
    }
};

// DPP controls (gfx9): quad permutations, and mirrors inside 8- and 16-lane rows.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 4, 8, 16, 32 or 64); every lane of a group
// ends with the same value (each butterfly step is symmetric).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    if constexpr (G >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (G >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (G >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (G >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// Maximum / sum over the 64 lanes of a wave, returned to every lane: an inclusive scan
// in registers (DPP shifts by 1, 2, 4 and 8 lanes within each 16-lane row, then
// row_bcast:15 and row_bcast:31 across rows; lanes without a source read the
// identity), whose total lane 63 holds.  Fixed order, so bit-reproducible.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or(float x, float identity) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, identity),
                                                                 __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_or<0x111, 0xF>(x, kNegInf));
    x = fmaxf(x, dpp_or<0x112, 0xF>(x, kNegInf));
    x = fmaxf(x, dpp_or<0x114, 0xF>(x, kNegInf));
    x = fmaxf(x, dpp_or<0x118, 0xF>(x, kNegInf));
    x = fmaxf(x, dpp_or<0x142, 0xA>(x, kNegInf));
    x = fmaxf(x, dpp_or<0x143, 0xC>(x, kNegInf));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_or<0x111, 0xF>(x, 0.f);
    x += dpp_or<0x112, 0xF>(x, 0.f);
    x += dpp_or<0x114, 0xF>(x, 0.f);
    x += dpp_or<0x118, 0xF>(x, 0.f);
    x += dpp_or<0x142, 0xA>(x, 0.f);
    x += dpp_or<0x143, 0xC>(x, 0.f);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
    return x;
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace tad
