// s6_fused.hip -- the Mamba-1 layer around the scan in one pass
// (ssm_s6_fused_fwd): causal depthwise conv1d + SiLU as the scan kernel's
// prologue, SiLU(z) gating as its epilogue (the FUSE instantiations of the
// kernel in s6_kernel.hpp), and the conv state the next call carries
// (conv_state.hpp).
//
// builderforce-memory-engine conv1d.ts (header, conv1d_forward) defines the
// causal depthwise convolution; mamba-rs 0.4.0 forward.rs F4a (conv1d
// burn-in with fused SiLU and a carried conv state), F4d (the scan) and F4e
// (gating) are the three launches this replaces.
#include "s6_kernel.hpp"
#include "conv_state.hpp"

namespace ssm {

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
    *kernel_name = "conv_state_out_kernel";
    if (a.bf16)
        launch_conv_state_out(static_cast<const uint16_t *>(a.x), a.conv_state, a.conv_state_out, a.batch, a.L,
                              a.d_inner, (int)a.d_conv, stream);
    else
        launch_conv_state_out(static_cast<const float *>(a.x), a.conv_state, a.conv_state_out, a.batch, a.L,
                              a.d_inner, (int)a.d_conv, stream);
    return hipGetLastError();
}

}  // namespace ssm
