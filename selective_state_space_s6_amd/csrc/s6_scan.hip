// s6_scan.hip -- the Mamba-1 (S6) forward selective scan of ssm_s6_scan_fwd:
// the plain instantiations of the kernel in s6_kernel.hpp.
#include "s6_kernel.hpp"

namespace ssm {

hipError_t launch_s6(const S6Args &a, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "s6_scan_kernel";
    S6Kp p{};
    p.u = a.u; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C;
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.Dm = a.d_inner; p.N = a.d_state;
    const int mode = (int)(a.flags & 0x3u);
    if (a.L == 1) {      // a decode step: one thread per channel (s6_decode.hip)
        S6FusedArgs f{a.u, nullptr, nullptr, nullptr, nullptr, a.dt, a.dt_bias, a.A_log, a.B, a.C, a.D, a.y,
                      a.h0, a.h_final, nullptr, nullptr, a.batch, a.L, a.d_inner, a.d_state, 1, a.bf16, a.flags};
        return launch_s6_step(f, false, stream, kernel_name);
    }
    if (a.workspace) {   // few channel blocks over a long sequence: time segments joined by a carry
        const S6SegPlan pl = s6_seg_plan(a.batch, a.L, a.d_inner, a.d_state);
        if (pl.nseg > 1) return launch_s6_segmented(a, pl, stream, kernel_name);
    }
    return a.bf16 ? launch_shape<uint16_t, false>(p, mode, stream) : launch_shape<float, false>(p, mode, stream);
}

hipError_t launch_s6_save(const S6Args &a, float *checkpoints, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "s6_scan_kernel";
    S6Kp p{};
    p.u = a.u; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C;
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.Dm = a.d_inner; p.N = a.d_state;
    p.ck = checkpoints;
    const int mode = (int)(a.flags & 0x3u);
    return a.bf16 ? launch_shape_save<uint16_t>(p, mode, stream) : launch_shape_save<float>(p, mode, stream);
}

}  // namespace ssm
