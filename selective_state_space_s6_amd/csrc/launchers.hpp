// launchers.hpp -- host-side kernel launchers behind the C interface.
// Arguments have been validated by abi.hip before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssm_scan.h"

namespace ssm {

struct S6Args {
    const void *u; const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; float *y;
    const float *h0; float *h_final;
    int64_t batch, L, d_inner, d_state;
    bool bf16; uint32_t flags;
    void *workspace = nullptr;   // at least s6_seg_plan(...).ws_bytes, or null: the sequential walk
};
hipError_t launch_s6(const S6Args &a, hipStream_t stream, const char **kernel_name);
// Segmented S6 scan (s6_seg.hip): long sequences over few channel blocks are cut
// into nseg time segments joined by an associative carry; nseg = 1 is the
// sequential walk.  ws_bytes: the workspace the segmented launch needs.
struct S6SegPlan { int64_t nseg, seg_len; size_t ws_bytes; };
S6SegPlan s6_seg_plan(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state);
hipError_t launch_s6_segmented(const S6Args &a, const S6SegPlan &plan, hipStream_t stream, const char **kernel_name);
// the forward that also writes the state entering every 16-step tile, (batch,
// ceil(L/16), d_inner, d_state) fp32, for the backward (d_state <= 16)
hipError_t launch_s6_save(const S6Args &a, float *checkpoints, hipStream_t stream, const char **kernel_name);
// B, C (batch, L, ngroups, d_state): channel d reads group d * ngroups / d_inner
// (one group goes to launch_s6)
hipError_t launch_s6_grouped(const S6Args &a, int64_t ngroups, hipStream_t stream, const char **kernel_name);
// launch_s6_grouped that also writes the state entering every 16-step tile to
// checkpoints (batch, ceil(L/16), d_inner, d_state); d_state <= 16
hipError_t launch_s6_grouped_save(const S6Args &a, int64_t ngroups, float *checkpoints, hipStream_t stream,
                                  const char **kernel_name);

// Mamba-1 layer around the scan: u = SiLU(causal conv1d(x)), y = scan(u) * SiLU(z)
struct S6FusedArgs {
    const void *x; const float *conv_w; const float *conv_b; const float *conv_state; const void *z;
    const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; float *y;
    const float *h0; float *h_final; float *u_out; float *conv_state_out;
    int64_t batch, L, d_inner, d_state, d_conv;
    bool bf16; uint32_t flags;
};
hipError_t launch_s6_fused(const S6FusedArgs &a, hipStream_t stream, const char **kernel_name);
// one step (L = 1) of either entry point; fused picks the conv + gate form
hipError_t launch_s6_step(const S6FusedArgs &a, bool fused, hipStream_t stream, const char **kernel_name);

// causal depthwise conv1d (+ SiLU) with a carried state (conv1d.hip)
struct Conv1dArgs {
    const void *x; const float *w; const float *bias; const float *state_in; void *y; float *state_out;
    int64_t batch, L, channels, d_conv;
    bool silu, bf16;
};
hipError_t launch_conv1d(const Conv1dArgs &a, hipStream_t stream, const char **kernel_name);

struct S6BwdArgs {
    const void *u; const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; const float *h0;
    const float *dy; const float *dh_final;
    float *du, *ddt, *dB, *dC, *dA_log, *dD, *ddt_bias, *dh0;
    int64_t batch, L, d_inner, d_state;
    bool bf16; uint32_t flags;
    void *workspace;
    const float *checkpoints = nullptr;   // the forward's saved states (batch, ceil(L/16), d_inner, d_state)
};
size_t s6_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state);
hipError_t launch_s6_bwd(const S6BwdArgs &a, hipStream_t stream, const char **kernel_name);
// the backward of launch_s6_grouped: dB, dC (batch, L, ngroups, d_state); d_state <= 16
size_t s6_grouped_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups);
hipError_t launch_s6_grouped_bwd(const S6BwdArgs &a, int64_t ngroups, hipStream_t stream, const char **kernel_name);

struct SsdArgs {
    const void *x; const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; float *y;
    const float *h0; float *h_final;
    int64_t batch, L, nheads, headdim, d_state, ngroups, chunk_len;
    bool bf16; uint32_t flags;
    void *workspace;
};
// The static device scratch of the entry points that allocate nothing (scratch.hip):
// kScratchBytes per GPU; scratch_address gives its address on the current device
// (looked up on the first call on each device).
constexpr size_t kScratchBytes = SSM_NOALLOC_SCRATCH_BYTES;
hipError_t scratch_address(void **out);

// one step (L = 1) of the SSD scan / its trapezoidal form (ssd_decode.hip)
hipError_t launch_ssd_step(const SsdArgs &a, hipStream_t stream, const char **kernel_name);

struct TrapRotArgs {
    const void *k_raw; const void *q_raw; const float *angles; const float *dt;
    const float *angle_state; void *k; void *q; float *angle_state_out;
    int64_t batch, L, nheads, d_state, n_angles;
    void *workspace;
};
size_t trap_rotate_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t d_state,
                                   int64_t n_angles);
hipError_t launch_trap_rotate(const TrapRotArgs &a, hipStream_t stream, const char **kernel_name);

struct SsdTrapArgs {
    const void *x; const void *k; const void *q;
    const float *dt; const float *a; const float *trap; const float *D; float *y;
    const float *h0; const void *k_prev; const void *x_prev; float *h_final;
    int64_t batch, L, nheads, headdim, d_state;
    void *workspace;
};
hipError_t launch_ssd_trap_step(const SsdTrapArgs &a, hipStream_t stream, const char **kernel_name);
size_t ssd_trap_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                int64_t d_state);
hipError_t launch_ssd_trap(const SsdTrapArgs &a, hipStream_t stream, const char **kernel_name);

struct SsdBwdArgs {
    const void *x; const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; const float *h0;
    const float *dy; const float *dh_final;
    float *dx, *ddt, *dB, *dC, *dA_log, *dD, *ddt_bias, *dh0;
    int64_t batch, L, nheads, headdim, d_state, ngroups;
    uint32_t flags;
    void *workspace;
};
size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                               int64_t d_state, int64_t ngroups);

// gradients of the Mamba-3 trapezoidal SSD (ssd_bwd.hip)
struct SsdTrapBwdArgs {
    const void *x; const void *k; const void *q;
    const float *dt; const float *a; const float *trap; const float *D; const float *h0;
    const void *k_prev; const void *x_prev; const float *dy; const float *dh_final;
    float *dx, *dk, *dq, *ddt, *da, *dtrap, *dD, *dh0, *dk_prev, *dx_prev;
    int64_t batch, L, nheads, headdim, d_state;
    void *workspace;
};
size_t ssd_trap_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state);
hipError_t launch_ssd_trap_bwd(const SsdTrapBwdArgs &a, hipStream_t stream, const char **kernel_name);
// the trapezoidal form's entering state h0' = h0 + dt_0 (1 - trap_0) x_prev (x) k_prev (ssd_scan.hip)
hipError_t launch_ssd_trap_h0(const void *x_prev, const void *k_prev, const float *dt, const float *trap,
                              const float *h0, float *h0p, int64_t batch, int64_t L, int64_t nheads,
                              int64_t headdim, int64_t d_state, hipStream_t stream);
hipError_t launch_ssd_bwd(const SsdBwdArgs &a, hipStream_t stream, const char **kernel_name);

size_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                           int64_t d_state, int64_t chunk_len);
hipError_t launch_ssd(const SsdArgs &a, hipStream_t stream, const char **kernel_name);

struct CssdArgs {
    const float *x; const float *dt; const float *dt_bias; const float *A_log;
    const float *B; const float *C; const float *D; float *y;
    const float *h0; float *h_final;
    int64_t batch, L, nheads, headdim, n_complex, ngroups, chunk_len;
    uint32_t flags;
    void *workspace;
    int64_t rank = 1;   // multi-input multi-output rank (a power of two, at most 16)
};
// L counts steps x rank for the multi-input multi-output form
size_t cssd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                            int64_t n_complex, int64_t chunk_len);
// work groups of the per-chunk preparation pass (must fit a launch)
int64_t cssd_prep_blocks(int64_t batch, int64_t L, int64_t nheads, int64_t ngroups);
hipError_t launch_cssd(const CssdArgs &a, hipStream_t stream, const char **kernel_name);

}  // namespace ssm
