// s6_fused.hip -- the Mamba-1 layer around the scan in one pass
// (ssm_s6_fused_fwd): causal depthwise conv1d + SiLU as the scan kernel's
// prologue, SiLU(z) gating as its epilogue (the FUSE instantiations of the
// kernel in s6_kernel.hpp), and the conv state the next call carries.
//
// builderforce-memory-engine conv1d.ts (header, conv1d_forward) defines the
// causal depthwise convolution; mamba-rs 0.4.0 forward.rs F4a (conv1d
// burn-in with fused SiLU and a carried conv state), F4d (the scan) and F4e
// (gating) are the three launches this replaces.
#include "s6_kernel.hpp"

namespace ssm {
namespace {

// conv_state_out[b, d, j] = x at time L-(K-1)+j, from the old state when that
// time is before 0.  One thread per (b, d) reads everything it needs before it
// writes, so the state may be updated in place; it runs after the scan, which
// reads the old state.
template <typename TIN>
__global__ void __launch_bounds__(256)
s6_conv_state_kernel(const TIN *x, const float *cs_in, float *cs_out, int64_t batch, int64_t L,
                     int64_t Dm, int K) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= batch * Dm) return;
    const int64_t b = i / Dm, d = i % Dm;
    float v[kMaxConv - 1];
#pragma unroll
    for (int j = 0; j < kMaxConv - 1; ++j) {
        if (j >= K - 1) break;
        const int64_t tt = L - (K - 1) + j;
        v[j] = tt >= 0 ? In<TIN>::ld(x, (b * L + tt) * Dm + d)
                       : (cs_in ? cs_in[i * (K - 1) + (K - 1) + tt] : 0.0f);
    }
#pragma unroll
    for (int j = 0; j < kMaxConv - 1; ++j) {
        if (j >= K - 1) break;
        cs_out[i * (K - 1) + j] = v[j];
    }
}

}  // namespace

hipError_t launch_s6_fused(const S6FusedArgs &a, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "s6_scan_kernel (fused)";
    S6Kp p{};
    p.u = a.x; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C;
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.Dm = a.d_inner; p.N = a.d_state;
    p.conv_w = a.conv_w; p.conv_b = a.conv_b; p.conv_state = a.conv_state; p.z = a.z;
    p.u_out = a.u_out; p.K = (int)a.d_conv;
    if (a.L == 1) return launch_s6_step(a, true, stream, kernel_name);   // a decode step
    const int mode = (int)(a.flags & 0x3u);
    hipError_t e = a.bf16 ? launch_shape<uint16_t, true>(p, mode, stream)
                          : launch_shape<float, true>(p, mode, stream);
    if (e != hipSuccess || a.conv_state_out == nullptr || a.d_conv < 2) return e;
    *kernel_name = "s6_conv_state_kernel";
    const int64_t n = a.batch * a.d_inner;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (a.bf16)
        hipLaunchKernelGGL(s6_conv_state_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t *>(a.x), a.conv_state, a.conv_state_out, a.batch, a.L,
                           a.d_inner, (int)a.d_conv);
    else
        hipLaunchKernelGGL(s6_conv_state_kernel<float>, grid, dim3(256), 0, stream,
                           static_cast<const float *>(a.x), a.conv_state, a.conv_state_out, a.batch, a.L,
                           a.d_inner, (int)a.d_conv);
    return hipGetLastError();
}

}  // namespace ssm
