// trap_rotate.hip -- Mamba-3 data-dependent rotation of k and q on gfx950.
//
// mamba-rs 0.2.1, src/mamba3_siso/gpu/mamba3_gpu.rs: F5 accumulates angle * dt
// step by step (per batch row, carried in the layer's angle state) and F4e+f
// rotates k and q by the accumulated angles.  Per (b, h) and angle j:
//   theta_t[j] = angle_state[b,h,j] + sum_{s<=t} angles[b,s,j] dt[b,s,h]
// and pair (2j, 2j+1) of k[b,t,h,:] and q[b,t,h,:] turns by theta_t[j]; pairs
// past n_angles are copied.
//
// The page's sequential accumulation runs one thread per (b, h, angle) over
// the whole sequence and stores every angle (B*T*nh*n_angles fp32) for the
// RoPE launch.  Here the sequence is cut into segments so the grid fills the
// chip, and no angle reaches HBM:
//   trap_rot_sums_kernel   one wave per (b, segment, h), lanes over angles:
//                          the segment's sum of angle * dt (and, in segment 0,
//                          a copy of the entering angle state, so that the
//                          state may be updated in place);
//   trap_rot_apply_kernel  same grid: the entering angle from the copy and the
//                          earlier segments' sums, then the segment's steps in
//                          order -- accumulate, sin/cos, rotate the bf16 pairs
//                          of k and q (fp32 arithmetic, one rounding to bf16),
//                          and the final angle from the last segment.
// Each step of a wave moves one k row and one q row of the head (N bf16 each,
// 4 bytes per lane), fully coalesced; loads run eight steps ahead.  When
// d_state % 8 == 0 and n_angles % 4 == 0 a vector variant moves 16 bytes per
// lane (four pairs, several heads per wave) and loads four steps ahead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "launchers.hpp"

namespace ssm {
namespace {

constexpr int kTargetWaves = 4096;   // 4 waves per SIMD
constexpr int kMinSeg = 64;          // shortest segment worth its own wave
constexpr int kAhead = 8;            // steps loaded ahead of the accumulation
constexpr int kAhead4 = 4;           // the same for the 16-byte vector path
constexpr int kGroupWaves = 8;       // head groups per work group (vector path)

struct RotKp {
    const uint32_t *k, *q;           // bf16 pairs
    const float *ang, *dt, *st_in;
    uint32_t *ko, *qo;
    float *st_out, *sums, *st_copy;
    int64_t batch, L, H, NP, NA, nseg, Ls;
};

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
// fp32 -> bf16, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void unit(const RotKp &p, int64_t &b, int64_t &seg, int64_t &h) {
    const int64_t blk = blockIdx.x;   // heads fastest: the heads of one segment share its angles
    h = blk % p.H;
    const int64_t bs = blk / p.H;
    seg = bs % p.nseg;
    b = bs / p.nseg;
}

__global__ void __launch_bounds__(64) trap_rot_sums_kernel(RotKp p) {
    int64_t b, seg, h;
    unit(p, b, seg, h);
    const int lane = threadIdx.x;
    const int64_t t0 = seg * p.Ls, n = min(p.Ls, p.L - t0);
    const float *dp = p.dt + (b * p.L + t0) * p.H + h;
    for (int64_t j = lane; j < p.NA; j += 64) {
        const float *ap = p.ang + (b * p.L + t0) * p.NA + j;
        float s = 0.0f;
        int64_t t = 0;
        for (; t + kAhead <= n; t += kAhead) {
            float av[kAhead], dv[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) {
                av[i] = ap[(t + i) * p.NA];
                dv[i] = dp[(t + i) * p.H];
            }
#pragma unroll
            for (int i = 0; i < kAhead; ++i) s = fmaf(av[i], dv[i], s);
        }
        for (; t < n; ++t) s = fmaf(ap[t * p.NA], dp[t * p.H], s);
        p.sums[((b * p.nseg + seg) * p.H + h) * p.NA + j] = s;
        if (seg == 0) {
            const int64_t o = (b * p.H + h) * p.NA + j;
            p.st_copy[o] = p.st_in ? p.st_in[o] : 0.0f;
        }
    }
}

// sin and cos of theta from the hardware's sin/cos, whose argument is in
// revolutions: theta / 2 pi reduced to [-1/2, 1/2] first.  The reduction's
// product carries ~6e-8 |theta| of rounding, as theta itself does in fp32;
// the results go to bf16 (2^-9 relative), far above either error.
__device__ __forceinline__ void sincos_rev(float th, float *s, float *c) {
    float r = th * 0.15915494309189535f;
    r -= rintf(r);
    *s = __builtin_amdgcn_sinf(r);
    *c = __builtin_amdgcn_cosf(r);
}

__device__ __forceinline__ uint32_t rotate_pair(uint32_t v, float c, float s) {
    const float x0 = bf_lo(v), x1 = bf_hi(v);
    const float y0 = fmaf(x0, c, -x1 * s);
    const float y1 = fmaf(x0, s, x1 * c);
    return to_bf16(y0) | (to_bf16(y1) << 16);
}

__global__ void __launch_bounds__(64) trap_rot_apply_kernel(RotKp p) {
    int64_t b, seg, h;
    unit(p, b, seg, h);
    const int lane = threadIdx.x;
    const int64_t t0 = seg * p.Ls, n = min(p.Ls, p.L - t0);
    const int64_t rs = p.H * p.NP;                       // row stride in pairs
    const float *dp = p.dt + (b * p.L + t0) * p.H + h;
    for (int64_t j = lane; j < p.NP; j += 64) {
        const bool rot = j < p.NA;
        const int64_t base = ((b * p.L + t0) * p.H + h) * p.NP + j;
        const uint32_t *kp = p.k + base, *qp = p.q + base;
        uint32_t *kop = p.ko + base, *qop = p.qo + base;
        if (!rot) {                                      // past the rotated pairs: copy
            for (int64_t t = 0; t < n; ++t) {
                kop[t * rs] = kp[t * rs];
                qop[t * rs] = qp[t * rs];
            }
            continue;
        }
        float th = p.st_copy[(b * p.H + h) * p.NA + j];
        for (int64_t s = 0; s < seg; ++s) th += p.sums[((b * p.nseg + s) * p.H + h) * p.NA + j];
        const float *ap = p.ang + (b * p.L + t0) * p.NA + j;
        int64_t t = 0;
        for (; t + kAhead <= n; t += kAhead) {
            float av[kAhead], dv[kAhead];
            uint32_t kv[kAhead], qv[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) {
                av[i] = ap[(t + i) * p.NA];
                dv[i] = dp[(t + i) * p.H];
                kv[i] = kp[(t + i) * rs];
                qv[i] = qp[(t + i) * rs];
            }
#pragma unroll
            for (int i = 0; i < kAhead; ++i) {
                th = fmaf(av[i], dv[i], th);
                float sn, cs;
                sincos_rev(th, &sn, &cs);
                kop[(t + i) * rs] = rotate_pair(kv[i], cs, sn);
                qop[(t + i) * rs] = rotate_pair(qv[i], cs, sn);
            }
        }
        for (; t < n; ++t) {
            th = fmaf(ap[t * p.NA], dp[t * p.H], th);
            float sn, cs;
            sincos_rev(th, &sn, &cs);
            kop[t * rs] = rotate_pair(kp[t * rs], cs, sn);
            qop[t * rs] = rotate_pair(qp[t * rs], cs, sn);
        }
        if (seg == p.nseg - 1 && p.st_out) p.st_out[(b * p.H + h) * p.NA + j] = th;
    }
}

// Vector path (d_state % 8 == 0, n_angles % 4 == 0): each lane moves 16 bytes
// of a row -- four pairs of k and of q, four angles -- so a wave covers
// 64 / lph heads of one step, lph = d_state / 8 lanes per head.  A lane's four
// pairs are either all rotated or all copied.
__device__ __forceinline__ void unit4(const RotKp &p, int64_t ngrp, int64_t &b, int64_t &seg, int64_t &hg) {
    // a work group holds gpb = blockDim.x / 64 consecutive head groups of one
    // (b, segment), so the group walks whole rows of k and q
    const int gpb = blockDim.x / 64;
    const int64_t nb = (ngrp + gpb - 1) / gpb;
    const int64_t blk = blockIdx.x;
    hg = (blk % nb) * gpb + threadIdx.x / 64;
    const int64_t bs = blk / nb;
    seg = bs % p.nseg;
    b = bs / p.nseg;
}

__global__ void __launch_bounds__(512) trap_rot_apply4_kernel(RotKp p, int lph, int hpw, int64_t ngrp) {
    int64_t b, seg, hg;
    unit4(p, ngrp, b, seg, hg);
    if (hg >= ngrp) return;                       // whole wave past the heads (no barrier)
    const int lane = threadIdx.x % 64;
    const int hl = lane / lph, jl = lane % lph;
    const int64_t h = hg * hpw + hl;
    if (hl >= hpw || h >= p.H) return;            // idle lanes (the kernel has no barrier)
    const int64_t t0 = seg * p.Ls, n = min(p.Ls, p.L - t0);
    const int64_t j0 = 4 * jl;
    const int64_t rs = p.H * p.NP / 4;            // row stride in 16-byte units
    const int64_t base = ((b * p.L + t0) * p.H + h) * (p.NP / 4) + jl;
    const uint4 *kp = reinterpret_cast<const uint4 *>(p.k) + base;
    const uint4 *qp = reinterpret_cast<const uint4 *>(p.q) + base;
    uint4 *kop = reinterpret_cast<uint4 *>(p.ko) + base;
    uint4 *qop = reinterpret_cast<uint4 *>(p.qo) + base;
    if (j0 >= p.NA) {                             // past the rotated pairs: copy
        for (int64_t t = 0; t < n; ++t) {
            kop[t * rs] = kp[t * rs];
            qop[t * rs] = qp[t * rs];
        }
        return;
    }
    const int64_t so = (b * p.H + h) * p.NA + j0;
    float4 th = *reinterpret_cast<const float4 *>(p.st_copy + so);
    for (int64_t s = 0; s < seg; ++s) {
        const float4 v = *reinterpret_cast<const float4 *>(p.sums + ((b * p.nseg + s) * p.H + h) * p.NA + j0);
        th.x += v.x; th.y += v.y; th.z += v.z; th.w += v.w;
    }
    const float4 *ap = reinterpret_cast<const float4 *>(p.ang + (b * p.L + t0) * p.NA + j0);
    const int64_t as = p.NA / 4;
    const float *dp = p.dt + (b * p.L + t0) * p.H + h;
    auto turn = [&](uint4 v, float4 c, float4 s) __attribute__((always_inline)) {
        return make_uint4(rotate_pair(v.x, c.x, s.x), rotate_pair(v.y, c.y, s.y),
                          rotate_pair(v.z, c.z, s.z), rotate_pair(v.w, c.w, s.w));
    };
    auto step = [&](float4 a, float d, uint4 kv, uint4 qv, int64_t t) __attribute__((always_inline)) {
        th.x = fmaf(a.x, d, th.x); th.y = fmaf(a.y, d, th.y);
        th.z = fmaf(a.z, d, th.z); th.w = fmaf(a.w, d, th.w);
        float4 sn, cs;
        sincos_rev(th.x, &sn.x, &cs.x); sincos_rev(th.y, &sn.y, &cs.y);
        sincos_rev(th.z, &sn.z, &cs.z); sincos_rev(th.w, &sn.w, &cs.w);
        kop[t * rs] = turn(kv, cs, sn);
        qop[t * rs] = turn(qv, cs, sn);
    };
    int64_t t = 0;
    for (; t + kAhead4 <= n; t += kAhead4) {
        float4 av[kAhead4];
        float dv[kAhead4];
        uint4 kv[kAhead4], qv[kAhead4];
#pragma unroll
        for (int i = 0; i < kAhead4; ++i) {
            av[i] = ap[(t + i) * as];
            dv[i] = dp[(t + i) * p.H];
            kv[i] = kp[(t + i) * rs];
            qv[i] = qp[(t + i) * rs];
        }
#pragma unroll
        for (int i = 0; i < kAhead4; ++i) step(av[i], dv[i], kv[i], qv[i], t + i);
    }
    for (; t < n; ++t) step(ap[t * as], dp[t * p.H], kp[t * rs], qp[t * rs], t);
    if (seg == p.nseg - 1 && p.st_out) *reinterpret_cast<float4 *>(p.st_out + so) = th;
}

// The segment sums in the vector path's layout (lanes over head x angle quad).
__global__ void __launch_bounds__(512) trap_rot_sums4_kernel(RotKp p, int lph, int hpw, int64_t ngrp) {
    int64_t b, seg, hg;
    unit4(p, ngrp, b, seg, hg);
    if (hg >= ngrp) return;
    const int lane = threadIdx.x % 64;
    const int hl = lane / lph, jl = lane % lph;
    const int64_t h = hg * hpw + hl, j0 = 4 * jl;
    if (hl >= hpw || h >= p.H || j0 >= p.NA) return;
    const int64_t t0 = seg * p.Ls, n = min(p.Ls, p.L - t0);
    const float4 *ap = reinterpret_cast<const float4 *>(p.ang + (b * p.L + t0) * p.NA + j0);
    const int64_t as = p.NA / 4;
    const float *dp = p.dt + (b * p.L + t0) * p.H + h;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int64_t t = 0;
    for (; t + kAhead <= n; t += kAhead) {
        float4 av[kAhead];
        float dv[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
            av[i] = ap[(t + i) * as];
            dv[i] = dp[(t + i) * p.H];
        }
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
            s.x = fmaf(av[i].x, dv[i], s.x); s.y = fmaf(av[i].y, dv[i], s.y);
            s.z = fmaf(av[i].z, dv[i], s.z); s.w = fmaf(av[i].w, dv[i], s.w);
        }
    }
    for (; t < n; ++t) {
        const float4 a = ap[t * as];
        const float d = dp[t * p.H];
        s.x = fmaf(a.x, d, s.x); s.y = fmaf(a.y, d, s.y);
        s.z = fmaf(a.z, d, s.z); s.w = fmaf(a.w, d, s.w);
    }
    *reinterpret_cast<float4 *>(p.sums + ((b * p.nseg + seg) * p.H + h) * p.NA + j0) = s;
    if (seg == 0) {
        const int64_t o = (b * p.H + h) * p.NA + j0;
        *reinterpret_cast<float4 *>(p.st_copy + o) =
            p.st_in ? *reinterpret_cast<const float4 *>(p.st_in + o) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
}

struct RotPlan {
    int64_t nseg, Ls;
};
// one wave per (batch, segment, unit), units = heads (scalar path) or head
// groups of the vector path
RotPlan rot_plan(int64_t batch, int64_t L, int64_t units) {
    int64_t nseg = (kTargetWaves + batch * units - 1) / (batch * units);
    nseg = std::max<int64_t>(1, std::min<int64_t>(nseg, (L + kMinSeg - 1) / kMinSeg));
    const int64_t Ls = (L + nseg - 1) / nseg;
    return RotPlan{(L + Ls - 1) / Ls, Ls};
}
bool vec_path(int64_t d_state, int64_t n_angles) { return d_state % 8 == 0 && n_angles % 4 == 0; }
// lanes per head and heads per wave of the vector path
int vec_lph(int64_t d_state) { return (int)(d_state / 8); }
int64_t plan_units(int64_t H, int64_t d_state, int64_t n_angles) {
    if (!vec_path(d_state, n_angles)) return H;
    const int hpw = 64 / vec_lph(d_state);
    return (H + hpw - 1) / hpw;
}
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

size_t trap_rotate_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t d_state,
                                   int64_t n_angles) {
    const RotPlan pl = rot_plan(batch, L, plan_units(nheads, d_state, n_angles));
    const int64_t na = n_angles > 0 ? n_angles : 1;
    return align256((size_t)(batch * pl.nseg * nheads * na) * sizeof(float)) +
           align256((size_t)(batch * nheads * na) * sizeof(float));
}

hipError_t launch_trap_rotate(const TrapRotArgs &a, hipStream_t stream, const char **kernel_name) {
    const int64_t units = plan_units(a.nheads, a.d_state, a.n_angles);
    const RotPlan pl = rot_plan(a.batch, a.L, units);
    RotKp p{};
    p.k = static_cast<const uint32_t *>(a.k_raw);
    p.q = static_cast<const uint32_t *>(a.q_raw);
    p.ang = a.angles; p.dt = a.dt; p.st_in = a.angle_state;
    p.ko = static_cast<uint32_t *>(a.k);
    p.qo = static_cast<uint32_t *>(a.q);
    p.st_out = a.angle_state_out;
    p.batch = a.batch; p.L = a.L; p.H = a.nheads; p.NP = a.d_state / 2; p.NA = a.n_angles;
    p.nseg = pl.nseg; p.Ls = pl.Ls;
    const int64_t na = a.n_angles > 0 ? a.n_angles : 1;
    char *ws = static_cast<char *>(a.workspace);
    p.sums = reinterpret_cast<float *>(ws);
    p.st_copy = reinterpret_cast<float *>(ws + align256((size_t)(a.batch * pl.nseg * a.nheads * na) * sizeof(float)));
    if (vec_path(a.d_state, a.n_angles)) {
        const int lph = vec_lph(a.d_state);
        const int64_t gpb = std::min<int64_t>(units, kGroupWaves);
        const dim3 grid((unsigned)(a.batch * pl.nseg * ((units + gpb - 1) / gpb))), block((unsigned)(64 * gpb));
        if (a.n_angles > 0) {
            *kernel_name = "trap_rot_sums4_kernel";
            hipLaunchKernelGGL(trap_rot_sums4_kernel, grid, block, 0, stream, p, lph, 64 / lph, units);
        }
        *kernel_name = "trap_rot_apply4_kernel";
        hipLaunchKernelGGL(trap_rot_apply4_kernel, grid, block, 0, stream, p, lph, 64 / lph, units);
    } else {
        if (a.n_angles > 0) {
            *kernel_name = "trap_rot_sums_kernel";
            hipLaunchKernelGGL(trap_rot_sums_kernel, dim3((unsigned)(a.batch * pl.nseg * a.nheads)), dim3(64),
                               0, stream, p);
        }
        *kernel_name = "trap_rot_apply_kernel";
        hipLaunchKernelGGL(trap_rot_apply_kernel, dim3((unsigned)(a.batch * pl.nseg * a.nheads)), dim3(64), 0,
                           stream, p);
    }
    return hipGetLastError();
}

}  // namespace ssm
