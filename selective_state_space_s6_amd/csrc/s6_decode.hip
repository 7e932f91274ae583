// s6_decode.hip -- one S6 step (L = 1): the decode step of ssm_s6_scan_fwd and
// ssm_s6_fused_fwd, with the state (and the conv state) carried in place.
//
// The scan kernel walks 16-step tiles for a VALU-bound sequence; a single
// step is bound by moving h (N floats per channel, read and written) and by
// latency.  Here a channel's states are spread over lanes in groups of four
// (float4 rows of h and A_log; N/4 lanes rounded up to a power of two), every
// lane forms u (conv + SiLU from the carried inputs in the fused form), the
// C.h terms are reduced by an xor tree, and the channel's first lane gates and
// writes y and the shifted conv state.  Every read of a state comes before its
// write, so h_final may be h0 and the conv state may be updated in place.
// Compute is not the bound, so the ZOH scale is the accurate
// delta * expm1(z) / z.  State sizes that are not a multiple of 4 take one
// thread per channel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launchers.hpp"

namespace ssm {
namespace {

constexpr int kMaxConvStep = 4;

// u of one step: conv + SiLU from the carried inputs (fused form), or x itself;
// old[] receives the carried inputs for the shifted state
template <typename TIN, bool FUSE>
__device__ __forceinline__ float step_input(const S6FusedArgs &a, int64_t i, int64_t d, float xv,
                                            float (&old)[kMaxConvStep - 1]) {
    if constexpr (!FUSE) {
        return xv;
    } else {
        const int K = (int)a.d_conv;
#pragma unroll
        for (int j = 0; j < kMaxConvStep - 1; ++j)
            old[j] = (j < K - 1 && a.conv_state) ? a.conv_state[i * (K - 1) + j] : 0.0f;
        float pre = fmaf(a.conv_w[d * K], xv, a.conv_b ? a.conv_b[d] : 0.0f);
#pragma unroll
        for (int k = 1; k < kMaxConvStep; ++k)   // x[t-k] is old[K-1-k]
            if (k < K) pre = fmaf(a.conv_w[d * K + k], old[K - 1 - k], pre);
        return silu_f(pre);
    }
}

// y, the gate, u_out and the shifted conv state of one channel
// (Dv and zv are loaded with the step's other inputs, before the reduction)
template <typename TIN, bool FUSE>
__device__ __forceinline__ void step_outputs(const S6FusedArgs &a, int64_t i, float xv, float uu, float ys,
                                             float Dv, float zv, const float (&old)[kMaxConvStep - 1]) {
    float y = fmaf(Dv, uu, ys);
    if constexpr (FUSE) {
        if (a.z) y *= silu_f(zv);
        if (a.u_out) a.u_out[i] = uu;
        const int K = (int)a.d_conv;
        if (a.conv_state_out) {
#pragma unroll
            for (int j = 0; j < kMaxConvStep - 1; ++j)
                if (j < K - 1) a.conv_state_out[i * (K - 1) + j] = j + 1 < K - 1 ? old[j + 1] : xv;
        }
    }
    a.y[i] = y;
}

// one state: Abar h + beta B u, and its C h term
template <int MODE>
__device__ __forceinline__ float step_state(float dl, float uu, float al, float hv, float bn, float cn, float &ys) {
    const float A = -expf(al);
    const float z = dl * A;
    float beta;
    if constexpr (MODE == 0) beta = z == 0.0f ? dl : dl * (expm1f(z) / z);
    else if constexpr (MODE == 1) beta = dl;
    else beta = 1.0f;
    const float hn = fmaf(expf(z), hv, beta * (bn * uu));
    ys = fmaf(cn, hn, ys);
    return hn;
}

// N % 4 == 0: 2^lg lanes per channel, lane q owns states 4q .. 4q+3 (float4 rows of
// h and A_log); C.h is reduced over the channel's lanes by an xor tree (fixed
// order).  Lanes past the states or past the last channel only take part in
// the shuffles.
template <typename TIN, int MODE, bool FUSE>
__global__ void __launch_bounds__(256) s6_step4_kernel(S6FusedArgs a, int lg) {
    const int64_t gt = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int lpc = 1 << lg;
    const int64_t i = gt >> lg;                           // (b, d) of the step
    const int q = (int)(gt & (lpc - 1));
    const int64_t N = a.d_state;
    const bool live = i < a.batch * a.d_inner;
    const int64_t ic = live ? i : 0;                      // clamped for the idle lanes' loads
    const int64_t b = ic / a.d_inner, d = ic % a.d_inner;
    const float xv = In<TIN>::ld(static_cast<const TIN *>(a.x), ic);
    const float Dv = a.D ? a.D[d] : 0.0f;
    const float zv = (FUSE && a.z) ? In<TIN>::ld(static_cast<const TIN *>(a.z), ic) : 0.0f;
    float old[kMaxConvStep - 1];
    const float uu = step_input<TIN, FUSE>(a, ic, d, xv, old);
    const float dl = softplus(a.dt[ic] + (a.dt_bias ? a.dt_bias[d] : 0.0f));
    float ys = 0.0f;
    const int64_t n = 4 * (int64_t)q;
    if (live && n < N) {
        const float4 al = *reinterpret_cast<const float4 *>(a.A_log + d * N + n);
        const float4 hv = a.h0 ? *reinterpret_cast<const float4 *>(a.h0 + ic * N + n)
                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const TIN *Bb = static_cast<const TIN *>(a.B) + b * N + n;
        const TIN *Cb = static_cast<const TIN *>(a.C) + b * N + n;
        float4 hn;
        hn.x = step_state<MODE>(dl, uu, al.x, hv.x, In<TIN>::ld(Bb, 0), In<TIN>::ld(Cb, 0), ys);
        hn.y = step_state<MODE>(dl, uu, al.y, hv.y, In<TIN>::ld(Bb, 1), In<TIN>::ld(Cb, 1), ys);
        hn.z = step_state<MODE>(dl, uu, al.z, hv.z, In<TIN>::ld(Bb, 2), In<TIN>::ld(Cb, 2), ys);
        hn.w = step_state<MODE>(dl, uu, al.w, hv.w, In<TIN>::ld(Bb, 3), In<TIN>::ld(Cb, 3), ys);
        if (a.h_final) *reinterpret_cast<float4 *>(a.h_final + ic * N + n) = hn;
    }
    for (int off = lpc >> 1; off > 0; off >>= 1) ys += __shfl_xor(ys, off, 64);
    if (live && q == 0) step_outputs<TIN, FUSE>(a, ic, xv, uu, ys, Dv, zv, old);
}

// any N: one thread per channel
template <typename TIN, int MODE, bool FUSE>
__global__ void __launch_bounds__(256) s6_step_kernel(S6FusedArgs a) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= a.batch * a.d_inner) return;
    const int64_t b = i / a.d_inner, d = i % a.d_inner, N = a.d_state;
    const float xv = In<TIN>::ld(static_cast<const TIN *>(a.x), i);
    const float Dv = a.D ? a.D[d] : 0.0f;
    const float zv = (FUSE && a.z) ? In<TIN>::ld(static_cast<const TIN *>(a.z), i) : 0.0f;
    float old[kMaxConvStep - 1];
    const float uu = step_input<TIN, FUSE>(a, i, d, xv, old);
    const float dl = softplus(a.dt[i] + (a.dt_bias ? a.dt_bias[d] : 0.0f));
    const TIN *Bb = static_cast<const TIN *>(a.B) + b * N;
    const TIN *Cb = static_cast<const TIN *>(a.C) + b * N;
    float ys = 0.0f;
    for (int64_t n = 0; n < N; ++n) {
        const float hn = step_state<MODE>(dl, uu, a.A_log[d * N + n], a.h0 ? a.h0[i * N + n] : 0.0f,
                                          In<TIN>::ld(Bb, n), In<TIN>::ld(Cb, n), ys);
        if (a.h_final) a.h_final[i * N + n] = hn;
    }
    step_outputs<TIN, FUSE>(a, i, xv, uu, ys, Dv, zv, old);
}

template <typename TIN, int MODE, bool FUSE>
void launch_v(const S6FusedArgs &a, hipStream_t s) {
    const int64_t n = a.batch * a.d_inner;
    if (a.d_state % 4 == 0) {
        int lg = 0;
        while ((4 << lg) < a.d_state) ++lg;               // 2^lg >= d_state / 4, at most 64 lanes
        const int64_t threads = n << lg;
        hipLaunchKernelGGL((s6_step4_kernel<TIN, MODE, FUSE>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, s, a, lg);
    } else {
        hipLaunchKernelGGL((s6_step_kernel<TIN, MODE, FUSE>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           a);
    }
}
template <typename TIN, bool FUSE>
void launch_m(const S6FusedArgs &a, hipStream_t s) {
    const int mode = (int)(a.flags & 0x3u);
    if (mode == 0) launch_v<TIN, 0, FUSE>(a, s);
    else if (mode == 1) launch_v<TIN, 1, FUSE>(a, s);
    else launch_v<TIN, 2, FUSE>(a, s);
}

}  // namespace

hipError_t launch_s6_step(const S6FusedArgs &a, bool fused, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "s6_step_kernel";
    if (a.bf16) {
        if (fused) launch_m<uint16_t, true>(a, stream);
        else launch_m<uint16_t, false>(a, stream);
    } else {
        if (fused) launch_m<float, true>(a, stream);
        else launch_m<float, false>(a, stream);
    }
    return hipGetLastError();
}

}  // namespace ssm
