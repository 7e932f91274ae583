// ssd_decode.hip -- one step (L = 1) of the SSD scan and of its Mamba-3
// trapezoidal form: the decode steps of ssd_chunk_scan_fwd and
// ssd_trap_chunk_scan_fwd, with the state carried in place.
//
// A step updates every element of the (headdim x d_state) fp32 state once:
//   SSD:  S = e^{a} S + sigma x (x) B,                      y = S C + D x
//   trap: S = alpha S + beta x_prev (x) k_prev + gamma x (x) k,   y = S q + D x
// so it is bound by reading and writing S.  One work group per (batch, head);
// a lane owns float4 chunks of state rows: a row's d_state/4 chunks sit on
// consecutive lanes (their count rounded up to a power of two, at most 64),
// the lanes' C.S terms are reduced by an xor tree in a fixed order, and the
// row's first lane writes y.  B (or k) and C (or q) of the lane's columns are
// loaded once.  Every element is read before it is written, so h_final may be
// h0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launchers.hpp"

namespace ssm {
namespace {

constexpr int kThreads = 256;

struct StepKp {
    const uint16_t *x, *B, *C, *x_prev, *k_prev;   // bf16
    const float *dt, *dt_bias, *A_log, *aval, *trap, *D, *h0;
    float *y, *h_final;
    int64_t batch, H, P, N, G;
    int mode;        // SSD input scale (flags bits 0-1)
    int lg;          // log2 of the lanes per state row
};

__device__ __forceinline__ float4 ld_bf16x4(const uint16_t *p) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}

template <bool TRAP>
__global__ void __launch_bounds__(kThreads) ssd_step_kernel(StepKp p) {
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int tid = threadIdx.x;
    const int lpr = 1 << p.lg;                     // lanes per state row
    const int rows = kThreads / lpr;               // rows per pass of the group
    const int c4 = tid & (lpr - 1);                // this lane's float4 chunk of a row
    const int64_t n = 4 * (int64_t)c4;
    const bool col = n < p.N;
    const int64_t o = b * p.H + h;                 // (b, 0, h): L = 1
    // per-head scalars of the step
    float dec, sig, gam = 0.0f, bet = 0.0f;
    if constexpr (TRAP) {
        const float dt = p.dt[o], tr = p.trap[o];
        dec = __expf(p.aval[o] * dt);              // alpha
        gam = tr * dt;
        bet = dec * dt * (1.0f - tr);
        sig = gam;
    } else {
        const float dl = softplus(p.dt[o] + (p.dt_bias ? p.dt_bias[h] : 0.0f));
        const float a = dl * (p.A_log ? -expf(p.A_log[h]) : 0.0f);
        dec = expf(a);
        sig = p.mode == 1 ? dl : p.mode == 2 ? 1.0f : (a == 0.0f ? dl : dl * (expm1f(a) / a));
    }
    const float Dh = p.D ? p.D[h] : 0.0f;
    // columns of this lane: B (or k), C (or q), and k_prev
    const int64_t g = TRAP ? h : h * p.G / p.H;
    const int64_t rowBC = (b * (TRAP ? p.H : p.G) + g) * p.N;
    float4 Bn = make_float4(0.0f, 0.0f, 0.0f, 0.0f), Cn = Bn, Kp = Bn;
    if (col) {
        Bn = ld_bf16x4(p.B + rowBC + n);
        Cn = ld_bf16x4(p.C + rowBC + n);
        if (TRAP && p.k_prev) Kp = ld_bf16x4(p.k_prev + o * p.N + n);
    }
    const int64_t sbase = o * p.P * p.N;           // (b, h) state
    for (int64_t r0 = 0; r0 < p.P; r0 += rows) {
        const int64_t r = r0 + tid / lpr;
        const bool live = r < p.P && col;
        const int64_t rc = r < p.P ? r : 0;
        const float xv = __uint_as_float((uint32_t)p.x[o * p.P + rc] << 16);
        float ys = 0.0f;
        if (live) {
            const float4 s = p.h0 ? *reinterpret_cast<const float4 *>(p.h0 + sbase + rc * p.N + n)
                                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            const float xs = sig * xv;
            float4 t = make_float4(fmaf(dec, s.x, xs * Bn.x), fmaf(dec, s.y, xs * Bn.y),
                                   fmaf(dec, s.z, xs * Bn.z), fmaf(dec, s.w, xs * Bn.w));
            if constexpr (TRAP) {
                if (p.x_prev) {
                    const float xp = bet * __uint_as_float((uint32_t)p.x_prev[o * p.P + rc] << 16);
                    t.x = fmaf(xp, Kp.x, t.x); t.y = fmaf(xp, Kp.y, t.y);
                    t.z = fmaf(xp, Kp.z, t.z); t.w = fmaf(xp, Kp.w, t.w);
                }
            }
            if (p.h_final) *reinterpret_cast<float4 *>(p.h_final + sbase + rc * p.N + n) = t;
            ys = fmaf(Cn.x, t.x, fmaf(Cn.y, t.y, fmaf(Cn.z, t.z, Cn.w * t.w)));
        }
        for (int off = lpr >> 1; off > 0; off >>= 1) ys += __shfl_xor(ys, off, 64);
        if (r < p.P && c4 == 0) p.y[o * p.P + r] = fmaf(Dh, xv, ys);
    }
}

int lanes_log2(int64_t N) {
    int lg = 0;
    while ((4 << lg) < N) ++lg;       // 2^lg >= N / 4; N <= 256 gives at most 64 lanes
    return lg;
}

}  // namespace

hipError_t launch_ssd_step(const SsdArgs &a, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "ssd_step_kernel";
    StepKp p{};
    p.x = static_cast<const uint16_t *>(a.x);
    p.B = static_cast<const uint16_t *>(a.B);
    p.C = static_cast<const uint16_t *>(a.C);
    p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.D = a.D; p.h0 = a.h0;
    p.y = a.y; p.h_final = a.h_final;
    p.batch = a.batch; p.H = a.nheads; p.P = a.headdim; p.N = a.d_state; p.G = a.ngroups;
    p.mode = (int)(a.flags & 0x3u);
    p.lg = lanes_log2(a.d_state);
    hipLaunchKernelGGL(ssd_step_kernel<false>, dim3((unsigned)(a.batch * a.nheads)), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_ssd_trap_step(const SsdTrapArgs &a, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "ssd_trap_step_kernel";
    StepKp p{};
    p.x = static_cast<const uint16_t *>(a.x);
    p.B = static_cast<const uint16_t *>(a.k);
    p.C = static_cast<const uint16_t *>(a.q);
    p.x_prev = static_cast<const uint16_t *>(a.x_prev);
    p.k_prev = static_cast<const uint16_t *>(a.k_prev);
    p.dt = a.dt; p.aval = a.a; p.trap = a.trap; p.D = a.D; p.h0 = a.h0;
    p.y = a.y; p.h_final = a.h_final;
    p.batch = a.batch; p.H = a.nheads; p.P = a.headdim; p.N = a.d_state; p.G = a.nheads;
    p.lg = lanes_log2(a.d_state);
    hipLaunchKernelGGL(ssd_step_kernel<true>, dim3((unsigned)(a.batch * a.nheads)), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ssm
