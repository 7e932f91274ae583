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

// Exact zero-order hold of one diagonal state with decay rate A < 0 over a
// step delta: Abar = e^z and beta = (e^z - 1)/A = delta * phi1(z), z = delta*A.
//
// The hardware exp2 is within 0.8 ulp, but e^z - 1 taken from it carries that
// rounding divided by |z|.  So where |z| >= 1/8, beta = (Abar - 1)/A (at most
// ~6 ulp); below, phi1 = (e^z - 1)/z comes from its degree-3 polynomial of
// least relative error on [-1/8, 0], written in x = z*log2(e) (fitted by
// Lawson's iteratively reweighted least squares; error 1.8e-8, < 1 ulp in fp32
// Horner form).  Abar is then formed on every lane as 1 + A*beta: where the
// series is used it carries no exp rounding at all, which matters because the
// slow states keep e^z's rounding for ~1/|z| steps (the hardware exp2 is biased
// by about -0.1 ulp near 1), and elsewhere it equals the hardware value to a
// few ulp of |Abar - 1|.  A, A*log2(e) and 1/A must be finite (|A| is clamped
// where it is formed).
constexpr float kZohSeriesX = 0.18033688f;   // 1/8 * log2(e): series below it
constexpr float kPhi1x1 = 0.34657156467437744f;
constexpr float kPhi1x2 = 0.08000794798135757f;
constexpr float kPhi1x3 = 0.01322636753320694f;
constexpr float kMaxAbsA = 1.0e38f;          // |A| clamp: A*log2(e) stays finite

struct Zoh {
    float ab;     // Abar = e^{delta A}
    float beta;   // (Abar - 1)/A
};
__device__ __forceinline__ Zoh zoh_exact(float dl, float A, float A2, float iA) {
    const float x = dl * A2;                                           // z * log2(e)
    const float e = exp2_fast(x);
    const float bf = fmaf(e, iA, -iA);                                 // (e^z - 1)/A
    const float p = fmaf(x, fmaf(x, fmaf(x, kPhi1x3, kPhi1x2), kPhi1x1), 1.0f);   // phi1
    const float beta = x > -kZohSeriesX ? dl * p : bf;
    return {fmaf(A, beta, 1.0f), beta};
}

// One state update h <- Abar h + beta b (b = B u) under the exact hold, where
// Abar = 1 + A beta_zoh.  With the ZOH input scale (beta = beta_zoh) it is
// h + beta (A h + b): two fused operations in which Abar is never rounded
// (rounded, Abar carries an absolute error of up to 2^-24 next to 1, the
// largest per-step error of a slowly decaying state).  With the other input
// scales (beta = delta or 1) Abar is taken as formed.
template <int MODE>
__device__ __forceinline__ float hold_step(float h, float ab, float A, float beta, float b) {
    if constexpr (MODE == 0) return fmaf(beta, fmaf(A, h, b), h);
    return fmaf(ab, h, beta * b);
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
