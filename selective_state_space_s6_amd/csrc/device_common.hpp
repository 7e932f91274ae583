// device_common.hpp -- small gfx950 device helpers shared by the scan kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_exp_f32: 2^x.  Inputs here are <= 0 or modest, so no range reduction is needed.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// v_log_f32: log2(x)
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// log(1 + e) for e in [0, 1], accurate also for tiny e: with w = 1 + e rounded,
// log1p(e) = log(w) * e / (w - 1) cancels the rounding of w (Goldberg's method).
__device__ __forceinline__ float log1p_small(float e) {
    const float w = 1.0f + e;
    const float d = w - 1.0f;
    return d == 0.0f ? e : log2_fast(w) * kLn2 * (e * __builtin_amdgcn_rcpf(d));
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}); no overflow for large x.
__device__ __forceinline__ float softplus(float x) {
    const float e = exp2_fast(-fabsf(x) * kLog2e);
    return fmaxf(x, 0.0f) + log1p_small(e);
}

// (e^z - 1)/z for z <= 0 and |z| < 1/16: Taylor polynomial, truncation < 2e-9.
__device__ __forceinline__ float phi1_small(float z) {
    float p = fmaf(z, 1.0f / 120.0f, 1.0f / 24.0f);
    p = fmaf(z, p, 1.0f / 6.0f);
    p = fmaf(z, p, 0.5f);
    return fmaf(z, p, 1.0f);
}

// SiLU(v) = v / (1 + e^-v), with the hardware reciprocal (about 1 ulp) in place of a
// division; for very negative v, e^-v overflows, its reciprocal is 0 and the result -0
__device__ __forceinline__ float silu_f(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// bf16 <-> fp32 (bf16 is the high half of an fp32 word)
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}
template <typename T> struct In;
template <> struct In<float> {
    __device__ __forceinline__ static float ld(const float *p, int64_t i) { return p[i]; }
};
template <> struct In<uint16_t> {
    __device__ __forceinline__ static float ld(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
};

// DPP row_newbcast:K -- every lane of a 16-lane row receives lane K of that row.
// update_dpp with old = 0 and bound_ctrl set lets the compiler fold the move
// into the consuming VOP2 instruction (v_mul_f32_dpp).
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0x150 + K, 0xf, 0xf, true));
}

// Inclusive prefix sum over each 32-lane half of a wave with DPP: row_shr 1,
// 2, 4, 8 with zero fill scans each 16-lane row, then row_bcast:15 adds the
// last lane of rows 0 and 2 to rows 1 and 3.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float scan32(float v) {
    v += dpp_f<0x111>(v);
    v += dpp_f<0x112>(v);
    v += dpp_f<0x114>(v);
    v += dpp_f<0x118>(v);
    v += dpp_f<0x142, 0xa>(v);
    return v;
}

// Block index -> work index such that consecutive work indices land on the
// same XCD (blocks are dealt round-robin over the 8 XCDs of an MI355X).
__device__ __forceinline__ int64_t xcd_swizzle(int64_t bid, int64_t nblk) {
    constexpr int64_t kXcd = 8;
    if (nblk % kXcd != 0) return bid;
    return (bid % kXcd) * (nblk / kXcd) + bid / kXcd;
}

}  // namespace ssm
