// abi.hip -- the extern "C" boundary of libssmscan.so (declared in
// include/ssm_scan.h): argument validation, workspace sizing, error strings,
// and dispatch to the kernel launchers.  Every check runs before any HIP call.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdarg.h>
#include <string.h>

#include "../../include/ssm_scan.h"
#include "launchers.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void *p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

#define REQUIRE_PTR(entry, p)                                                        \
    do {                                                                             \
        if ((p) == nullptr) return fail(SSM_ERR_INVALID_ARG, "%s: %s is NULL", entry, #p); \
    } while (0)
#define REQUIRE_POS(entry, v)                                                                  \
    do {                                                                                       \
        if ((v) <= 0) return fail(SSM_ERR_INVALID_ARG, "%s: %s must be > 0 (got %lld)", entry, \
                                  #v, (long long)(v));                                         \
    } while (0)
#define REQUIRE_ALIGN(entry, p)                                                                 \
    do {                                                                                        \
        if (!aligned16(p)) return fail(SSM_ERR_UNSUPPORTED, "%s: %s is not 16-byte aligned", \
                                       entry, #p);                                              \
    } while (0)

int launched(const char *entry, hipError_t e, const char *kernel) {
    if (e != hipSuccess)
        return fail(SSM_ERR_HIP, "%s: launch of %s failed: %s", entry, kernel, hipGetErrorString(e));
    g_err[0] = '\0';
    return SSM_OK;
}

// elements of a tensor must stay addressable with 64-bit offsets and the grid
// with 32-bit block counts
bool too_big(int64_t a, int64_t b, int64_t c, int64_t d) {
    const double n = (double)a * (double)b * (double)c * (double)d;
    return n > 9.0e15;
}

}  // namespace

extern "C" {

const char *ssm_last_error(void) { return g_err; }

size_t ssm_s6_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state) {
    if (batch <= 0 || L <= 0 || d_inner <= 0 || d_state <= 0) return 0;
    return ssm::s6_seg_plan(batch, L, d_inner, d_state).ws_bytes;
}

int ssm_s6_scan_fwd(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                    const void *B, const void *C, const float *D, float *y,
                    const float *h0, float *h_final,
                    int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                    ssm_dtype_t in_dtype, uint32_t flags,
                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssm_s6_scan_fwd";
    REQUIRE_PTR(E, u); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, y);
    REQUIRE_POS(E, batch); REQUIRE_POS(E, L); REQUIRE_POS(E, d_inner); REQUIRE_POS(E, d_state);
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if ((flags & ~0x3u) != 0 || (flags & 0x3u) == 0x3u)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x: only SSM_BBAR_ZOH/DT/ONE apply", E, flags);
    if (d_state > SSM_MAX_D_STATE)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld > %d", E, (long long)d_state, SSM_MAX_D_STATE);
    if (too_big(batch, L, d_inner, 1) || batch * ((d_inner + 255) / 16) > 0x7fffffffLL)
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    REQUIRE_ALIGN(E, u); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, y);
    REQUIRE_ALIGN(E, h0); REQUIRE_ALIGN(E, h_final);
    if ((const void *)y == u || (const void *)y == (const void *)dt || (const void *)y == B ||
        (const void *)y == C)
        return fail(SSM_ERR_INVALID_ARG, "%s: y aliases an input", E);
    // the workspace is optional: with one of at least the queried size, long
    // sequences over few channels take the segmented scan; without, the walk
    const size_t need = ssm::s6_seg_plan(batch, L, d_inner, d_state).ws_bytes;
    if (workspace && workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", E, workspace_bytes, need);
    REQUIRE_ALIGN(E, workspace);
    ssm::S6Args a{u, dt, dt_bias, A_log, B, C, D, y, h0, h_final, batch, L, d_inner, d_state,
                  in_dtype == SSM_BF16, flags, need > 0 ? workspace : nullptr};
    const char *kn = "s6";
    return launched(E, ssm::launch_s6(a, stream, &kn), kn);
}

size_t ssm_s6_scan_checkpoint_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state) {
    if (batch <= 0 || L <= 0 || d_inner <= 0 || d_state <= 0) return 0;
    return (size_t)(batch * ((L + 15) / 16) * d_inner * d_state) * sizeof(float);
}

static int s6_fwd_save_call(const char *E, int64_t ngroups, const void *u, const float *dt, const float *dt_bias,
                            const float *A_log, const void *B, const void *C, const float *D, float *y,
                            const float *h0, float *h_final, float *checkpoints,
                            int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                            ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream) {
    REQUIRE_PTR(E, u); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, y); REQUIRE_PTR(E, checkpoints);
    REQUIRE_POS(E, batch); REQUIRE_POS(E, L); REQUIRE_POS(E, d_inner); REQUIRE_POS(E, d_state);
    REQUIRE_POS(E, ngroups);
    if (d_inner % ngroups != 0)
        return fail(SSM_ERR_INVALID_ARG, "%s: d_inner %lld is not a multiple of ngroups %lld", E,
                    (long long)d_inner, (long long)ngroups);
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if ((flags & ~0x3u) != 0 || (flags & 0x3u) == 0x3u)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x: only SSM_BBAR_ZOH/DT/ONE apply", E, flags);
    if (d_state > SSM_S6_BWD_MAX_D_STATE)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld > %d (the backward's limit)", E, (long long)d_state,
                    SSM_S6_BWD_MAX_D_STATE);
    if (too_big(batch, L, d_inner, 1) || too_big(batch, (L + 15) / 16, d_inner, d_state) ||
        too_big(batch, L, ngroups, d_state) || batch * ((d_inner + 255) / 16) > 0x7fffffffLL)
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    REQUIRE_ALIGN(E, u); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, y);
    REQUIRE_ALIGN(E, h0); REQUIRE_ALIGN(E, h_final); REQUIRE_ALIGN(E, checkpoints);
    const void *ins[] = {u, dt, dt_bias, A_log, B, C, D, h0};
    for (const void *o : {(const void *)y, (const void *)checkpoints})
        for (const void *in : ins)
            if (o == in) return fail(SSM_ERR_INVALID_ARG, "%s: an output aliases an input", E);
    if ((const void *)y == (const void *)checkpoints || (const void *)h_final == (const void *)checkpoints ||
        (const void *)h_final == (const void *)y)
        return fail(SSM_ERR_INVALID_ARG, "%s: two outputs alias", E);
    ssm::S6Args a{u, dt, dt_bias, A_log, B, C, D, y, h0, h_final, batch, L, d_inner, d_state,
                  in_dtype == SSM_BF16, flags};
    const char *kn = "s6_save";
    return launched(E, ssm::launch_s6_grouped_save(a, ngroups, checkpoints, stream, &kn), kn);
}

int ssm_s6_scan_fwd_save(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                         const void *B, const void *C, const float *D, float *y,
                         const float *h0, float *h_final, float *checkpoints,
                         int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                         ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream) {
    return s6_fwd_save_call("ssm_s6_scan_fwd_save", 1, u, dt, dt_bias, A_log, B, C, D, y, h0, h_final,
                            checkpoints, batch, L, d_inner, d_state, in_dtype, flags, stream);
}

int ssm_s6_scan_grouped_fwd_save(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                                 const void *B, const void *C, const float *D, float *y,
                                 const float *h0, float *h_final, float *checkpoints,
                                 int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                                 ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream) {
    return s6_fwd_save_call("ssm_s6_scan_grouped_fwd_save", ngroups, u, dt, dt_bias, A_log, B, C, D, y, h0,
                            h_final, checkpoints, batch, L, d_inner, d_state, in_dtype, flags, stream);
}

int ssm_s6_scan_grouped_fwd(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                            const void *B, const void *C, const float *D, float *y,
                            const float *h0, float *h_final,
                            int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                            ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream) {
    const char *E = "ssm_s6_scan_grouped_fwd";
    REQUIRE_PTR(E, u); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, y);
    REQUIRE_POS(E, batch); REQUIRE_POS(E, L); REQUIRE_POS(E, d_inner); REQUIRE_POS(E, d_state);
    REQUIRE_POS(E, ngroups);
    if (d_inner % ngroups != 0)
        return fail(SSM_ERR_INVALID_ARG, "%s: d_inner %lld is not a multiple of ngroups %lld", E,
                    (long long)d_inner, (long long)ngroups);
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if ((flags & ~0x3u) != 0 || (flags & 0x3u) == 0x3u)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x: only SSM_BBAR_ZOH/DT/ONE apply", E, flags);
    if (d_state > (ngroups == 1 ? SSM_MAX_D_STATE : SSM_MAX_D_STATE_GROUPED))
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld > %d", E, (long long)d_state,
                    ngroups == 1 ? SSM_MAX_D_STATE : SSM_MAX_D_STATE_GROUPED);
    if (too_big(batch, L, d_inner, 1) || too_big(batch, L, ngroups, d_state) ||
        batch * ((d_inner + 255) / 16) > 0x7fffffffLL)
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    REQUIRE_ALIGN(E, u); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, y);
    REQUIRE_ALIGN(E, h0); REQUIRE_ALIGN(E, h_final);
    if ((const void *)y == u || (const void *)y == (const void *)dt || (const void *)y == B ||
        (const void *)y == C)
        return fail(SSM_ERR_INVALID_ARG, "%s: y aliases an input", E);
    ssm::S6Args a{u, dt, dt_bias, A_log, B, C, D, y, h0, h_final, batch, L, d_inner, d_state,
                  in_dtype == SSM_BF16, flags};
    const char *kn = "s6_grouped";
    return launched(E, ssm::launch_s6_grouped(a, ngroups, stream, &kn), kn);
}

int ssm_s6_fused_fwd(const void *x, const float *conv_w, const float *conv_b, const float *conv_state,
                     const void *z, const float *dt, const float *dt_bias, const float *A_log,
                     const void *B, const void *C, const float *D, float *y,
                     const float *h0, float *h_final, float *u_out, float *conv_state_out,
                     int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t d_conv,
                     ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream) {
    const char *E = "ssm_s6_fused_fwd";
    REQUIRE_PTR(E, x); REQUIRE_PTR(E, conv_w); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, y);
    REQUIRE_POS(E, batch); REQUIRE_POS(E, L); REQUIRE_POS(E, d_inner); REQUIRE_POS(E, d_state);
    REQUIRE_POS(E, d_conv);
    if (d_conv > SSM_MAX_D_CONV)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_conv %lld > %d", E, (long long)d_conv, SSM_MAX_D_CONV);
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if ((flags & ~0x3u) != 0 || (flags & 0x3u) == 0x3u)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x: only SSM_BBAR_ZOH/DT/ONE apply", E, flags);
    if (d_state > SSM_MAX_D_STATE)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld > %d", E, (long long)d_state, SSM_MAX_D_STATE);
    if (too_big(batch, L, d_inner, 1) || batch * ((d_inner + 255) / 16) > 0x7fffffffLL)
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    REQUIRE_ALIGN(E, x); REQUIRE_ALIGN(E, conv_w); REQUIRE_ALIGN(E, conv_b); REQUIRE_ALIGN(E, conv_state);
    REQUIRE_ALIGN(E, z); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, y);
    REQUIRE_ALIGN(E, h0); REQUIRE_ALIGN(E, h_final); REQUIRE_ALIGN(E, u_out); REQUIRE_ALIGN(E, conv_state_out);
    // h_final may be h0 and conv_state_out may be conv_state (carried in place);
    // no other output may share memory with an input or another output
    {
        const void *ins[] = {x, conv_w, conv_b, conv_state, z, dt, dt_bias, A_log, B, C, D, h0};
        const void *outs[] = {y, h_final, u_out, conv_state_out};
        for (size_t i = 0; i < 4; ++i) {
            if (!outs[i]) continue;
            for (const void *in : ins)
                if (in == outs[i] && !(i == 1 && in == (const void *)h0) && !(i == 3 && in == (const void *)conv_state))
                    return fail(SSM_ERR_INVALID_ARG, "%s: an output aliases an input", E);
            for (size_t j = 0; j < i; ++j)
                if (outs[j] == outs[i]) return fail(SSM_ERR_INVALID_ARG, "%s: two outputs alias", E);
        }
    }
    ssm::S6FusedArgs a{x, conv_w, conv_b, conv_state, z, dt, dt_bias, A_log, B, C, D, y, h0, h_final, u_out,
                       conv_state_out, batch, L, d_inner, d_state, d_conv, in_dtype == SSM_BF16, flags};
    const char *kn = "s6_fused";
    return launched(E, ssm::launch_s6_fused(a, stream, &kn), kn);
}

int ssm_causal_conv1d_fwd(const void *x, const float *w, const float *bias, const float *state_in, void *y,
                          float *state_out, int64_t batch, int64_t L, int64_t channels, int64_t d_conv,
                          int silu, ssm_dtype_t dtype, hipStream_t stream) {
    const char *E = "ssm_causal_conv1d_fwd";
    REQUIRE_PTR(E, x); REQUIRE_PTR(E, w); REQUIRE_PTR(E, y);
    REQUIRE_POS(E, batch); REQUIRE_POS(E, L); REQUIRE_POS(E, channels); REQUIRE_POS(E, d_conv);
    if (d_conv > SSM_MAX_D_CONV)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_conv %lld > %d", E, (long long)d_conv, SSM_MAX_D_CONV);
    if (silu != 0 && silu != 1) return fail(SSM_ERR_INVALID_ARG, "%s: silu must be 0 or 1 (got %d)", E, silu);
    if (dtype != SSM_F32 && dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: dtype %d is not SSM_F32 or SSM_BF16", E, (int)dtype);
    if (too_big(batch, L, channels, 1) || batch * ((L + 31) / 32) * channels > 0x7fffffffLL * 256)
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    REQUIRE_ALIGN(E, x); REQUIRE_ALIGN(E, w); REQUIRE_ALIGN(E, bias); REQUIRE_ALIGN(E, state_in);
    REQUIRE_ALIGN(E, y); REQUIRE_ALIGN(E, state_out);
    {
        const void *ins[] = {x, w, bias, state_in};
        for (const void *in : ins)
            if (in && in == y) return fail(SSM_ERR_INVALID_ARG, "%s: y aliases an input", E);
        const void *others[] = {x, w, bias, y};
        for (const void *o : others)
            if (state_out && o == (const void *)state_out)
                return fail(SSM_ERR_INVALID_ARG, "%s: state_out aliases another argument", E);
    }
    ssm::Conv1dArgs a{x, w, bias, state_in, y, state_out, batch, L, channels, d_conv, silu == 1, dtype == SSM_BF16};
    const char *kn = "conv1d";
    return launched(E, ssm::launch_conv1d(a, stream, &kn), kn);
}

size_t ssm_s6_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state) {
    if (batch <= 0 || L <= 0 || d_inner <= 0 || d_state <= 0) return 0;
    return ssm::s6_bwd_workspace_bytes(batch, L, d_inner, d_state);
}

static int s6_bwd_call(const char *E, int64_t ngroups, const void *u, const float *dt, const float *dt_bias,
                       const float *A_log, const void *B, const void *C, const float *D, const float *h0,
                       const float *dy, const float *dh_final, const float *checkpoints,
                       float *du, float *ddt, float *dB, float *dC, float *dA_log,
                       float *dD, float *ddt_bias, float *dh0,
                       int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                       ssm_dtype_t in_dtype, uint32_t flags,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    REQUIRE_PTR(E, u); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, dy);
    REQUIRE_PTR(E, du); REQUIRE_PTR(E, ddt); REQUIRE_PTR(E, dB); REQUIRE_PTR(E, dC);
    REQUIRE_PTR(E, dA_log);
    REQUIRE_POS(E, batch); REQUIRE_POS(E, L); REQUIRE_POS(E, d_inner); REQUIRE_POS(E, d_state);
    REQUIRE_POS(E, ngroups);
    if (d_inner % ngroups != 0)
        return fail(SSM_ERR_INVALID_ARG, "%s: d_inner %lld is not a multiple of ngroups %lld", E,
                    (long long)d_inner, (long long)ngroups);
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if ((flags & ~0x3u) != 0 || (flags & 0x3u) == 0x3u)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x: only SSM_BBAR_ZOH/DT/ONE apply", E, flags);
    if (d_state > SSM_S6_BWD_MAX_D_STATE)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld > %d", E, (long long)d_state,
                    SSM_S6_BWD_MAX_D_STATE);
    if ((ngroups > 1 && (too_big(batch, L, d_inner, d_state) ||   // the per-channel dB, dC shares
                         d_inner * d_state >= (1LL << 26))) ||     // the grouped kernel's 32-bit offsets
        too_big(batch, L, d_inner, 1) || too_big(batch, (L + 15) / 16, d_inner, d_state) ||
        batch * ((d_inner + 15) / 16) > 0x7fffffffLL || L > 0x7fffffefLL || d_inner >= (1LL << 25))
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    REQUIRE_ALIGN(E, u); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, h0);
    REQUIRE_ALIGN(E, dy); REQUIRE_ALIGN(E, dh_final);
    REQUIRE_ALIGN(E, du); REQUIRE_ALIGN(E, ddt); REQUIRE_ALIGN(E, dB); REQUIRE_ALIGN(E, dC);
    REQUIRE_ALIGN(E, dA_log); REQUIRE_ALIGN(E, dD); REQUIRE_ALIGN(E, ddt_bias); REQUIRE_ALIGN(E, dh0);
    REQUIRE_ALIGN(E, workspace);
    REQUIRE_ALIGN(E, checkpoints);
    const void *ins[] = {u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, workspace, checkpoints};
    const void *outs[] = {du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        if (outs[i] == nullptr) continue;
        for (size_t j = 0; j < sizeof(ins) / sizeof(ins[0]); ++j)
            if (outs[i] == ins[j]) return fail(SSM_ERR_INVALID_ARG, "%s: an output aliases an input", E);
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (outs[i] == outs[j]) return fail(SSM_ERR_INVALID_ARG, "%s: two outputs alias", E);
    }
    const size_t need = ssm::s6_grouped_bwd_workspace_bytes(batch, L, d_inner, d_state, ngroups);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", E, need,
                    workspace ? workspace_bytes : (size_t)0);
    ssm::S6BwdArgs a{u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final,
                     du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0,
                     batch, L, d_inner, d_state, in_dtype == SSM_BF16, flags, workspace, checkpoints};
    const char *kn = "s6_bwd";
    return launched(E, ssm::launch_s6_grouped_bwd(a, ngroups, stream, &kn), kn);
}


int ssm_s6_scan_bwd(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                    const void *B, const void *C, const float *D, const float *h0,
                    const float *dy, const float *dh_final,
                    float *du, float *ddt, float *dB, float *dC, float *dA_log,
                    float *dD, float *ddt_bias, float *dh0,
                    int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                    ssm_dtype_t in_dtype, uint32_t flags,
                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return s6_bwd_call("ssm_s6_scan_bwd", 1, u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, nullptr,
                       du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0, batch, L, d_inner, d_state, in_dtype, flags,
                       workspace, workspace_bytes, stream);
}

size_t ssm_s6_scan_grouped_bwd_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                              int64_t ngroups) {
    if (batch <= 0 || L <= 0 || d_inner <= 0 || d_state <= 0 || ngroups <= 0) return 0;
    return ssm::s6_grouped_bwd_workspace_bytes(batch, L, d_inner, d_state, ngroups);
}

int ssm_s6_scan_grouped_bwd(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                            const void *B, const void *C, const float *D, const float *h0,
                            const float *dy, const float *dh_final,
                            float *du, float *ddt, float *dB, float *dC, float *dA_log,
                            float *dD, float *ddt_bias, float *dh0,
                            int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                            ssm_dtype_t in_dtype, uint32_t flags,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return s6_bwd_call("ssm_s6_scan_grouped_bwd", ngroups, u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final,
                       nullptr, du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0, batch, L, d_inner, d_state, in_dtype,
                       flags, workspace, workspace_bytes, stream);
}

int ssm_s6_scan_grouped_bwd_saved(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                                  const void *B, const void *C, const float *D, const float *h0,
                                  const float *dy, const float *dh_final, const float *checkpoints,
                                  float *du, float *ddt, float *dB, float *dC, float *dA_log,
                                  float *dD, float *ddt_bias, float *dh0,
                                  int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                                  ssm_dtype_t in_dtype, uint32_t flags,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssm_s6_scan_grouped_bwd_saved";
    REQUIRE_PTR(E, checkpoints);
    return s6_bwd_call(E, ngroups, u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, checkpoints,
                       du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0, batch, L, d_inner, d_state, in_dtype, flags,
                       workspace, workspace_bytes, stream);
}

int ssm_s6_scan_bwd_saved(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                          const void *B, const void *C, const float *D, const float *h0,
                          const float *dy, const float *dh_final, const float *checkpoints,
                          float *du, float *ddt, float *dB, float *dC, float *dA_log,
                          float *dD, float *ddt_bias, float *dh0,
                          int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                          ssm_dtype_t in_dtype, uint32_t flags,
                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssm_s6_scan_bwd_saved";
    REQUIRE_PTR(E, checkpoints);
    return s6_bwd_call(E, 1, u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, checkpoints,
                       du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0, batch, L, d_inner, d_state, in_dtype, flags,
                       workspace, workspace_bytes, stream);
}

static int ssd_check_shape(const char *E, int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                           int64_t d_state, int64_t ngroups, int64_t chunk_len) {
    REQUIRE_POS(E, batch); REQUIRE_POS(E, L); REQUIRE_POS(E, nheads); REQUIRE_POS(E, headdim);
    REQUIRE_POS(E, d_state); REQUIRE_POS(E, ngroups); REQUIRE_POS(E, chunk_len);
    if (nheads % ngroups != 0)
        return fail(SSM_ERR_INVALID_ARG, "%s: nheads %lld is not a multiple of ngroups %lld", E,
                    (long long)nheads, (long long)ngroups);
    if (too_big(batch, L, nheads, headdim) || too_big(batch, L, ngroups, d_state))
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    // a chunk's rows are addressed by 32-bit byte offsets from a per-chunk base
    if (nheads * headdim > (1LL << 24))
        return fail(SSM_ERR_UNSUPPORTED, "%s: nheads * headdim %lld exceeds 2^24", E,
                    (long long)(nheads * headdim));
    return SSM_OK;
}

size_t ssd_chunk_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                         int64_t d_state, int64_t ngroups, int64_t chunk_len) {
    (void)ngroups;
    if (batch <= 0 || L <= 0 || nheads <= 0 || headdim <= 0 || d_state <= 0 || chunk_len <= 0) return 0;
    return ssm::ssd_workspace_bytes(batch, L, nheads, headdim, d_state, chunk_len);
}

}  // extern "C"

namespace {
// ssd_chunk_scan_fwd and its no-allocation form: every check before any HIP call;
// scratch: the workspace is the library's static device scratch
int ssd_fwd_call(const char *E, const void *x, const float *dt, const float *dt_bias, const float *A_log,
                 const void *B, const void *C, const float *D, float *y, const float *h0, float *h_final,
                 int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                 int64_t ngroups, int64_t chunk_len, ssm_dtype_t in_dtype, uint32_t flags,
                 void *workspace, size_t workspace_bytes, hipStream_t stream, bool scratch) {
    REQUIRE_PTR(E, x); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, y);
    int rc = ssd_check_shape(E, batch, L, nheads, headdim, d_state, ngroups, chunk_len);
    if (rc != SSM_OK) return rc;
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if (in_dtype != SSM_BF16)
        return fail(SSM_ERR_UNSUPPORTED, "%s: the MFMA path takes bf16 x, B, C (SSM_BF16)", E);
    if ((flags & ~0x3u) != 0 || (flags & 0x3u) == 0x3u)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x: only SSM_BBAR_ZOH/DT/ONE apply", E, flags);
    if (!(headdim == 32 || headdim == 64 || headdim == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: headdim %lld not in {32, 64, 128}", E, (long long)headdim);
    if (d_state % 32 != 0 || d_state > SSM_MAX_D_STATE)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld must be a multiple of 32 and <= %d", E,
                    (long long)d_state, SSM_MAX_D_STATE);
    if (!(chunk_len == 64 || chunk_len == 128 || chunk_len == 256))
        return fail(SSM_ERR_UNSUPPORTED, "%s: chunk_len %lld not in {64, 128, 256}", E, (long long)chunk_len);
    REQUIRE_ALIGN(E, x); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, y);
    REQUIRE_ALIGN(E, h0); REQUIRE_ALIGN(E, h_final); REQUIRE_ALIGN(E, workspace);
    if ((const void *)y == x || (const void *)y == (const void *)dt || (const void *)y == B ||
        (const void *)y == C)
        return fail(SSM_ERR_INVALID_ARG, "%s: y aliases an input", E);
    const size_t need = ssm::ssd_workspace_bytes(batch, L, nheads, headdim, d_state, chunk_len);
    if (scratch) {
        if (need > ssm::kScratchBytes)
            return fail(SSM_ERR_WORKSPACE, "%s: this shape needs %zu bytes of segment states, more than the "
                        "%zu-byte static scratch (ssd_chunk_scan_fwd takes a caller workspace)", E, need,
                        ssm::kScratchBytes);
        if (need > 0) {
            const hipError_t e = ssm::scratch_address(&workspace);
            if (e != hipSuccess)
                return fail(SSM_ERR_HIP, "%s: address of the static scratch: %s", E, hipGetErrorString(e));
            workspace_bytes = ssm::kScratchBytes;
        }
    } else if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", E, need,
                    workspace ? workspace_bytes : (size_t)0);
    }
    ssm::SsdArgs a{x, dt, dt_bias, A_log, B, C, D, y, h0, h_final, batch, L, nheads, headdim,
                   d_state, ngroups, chunk_len, in_dtype == SSM_BF16, flags, workspace};
    const char *kn = "ssd";
    return launched(E, ssm::launch_ssd(a, stream, &kn), kn);
}
}  // namespace

extern "C" {

int ssd_chunk_scan_fwd(const void *x, const float *dt, const float *dt_bias, const float *A_log,
                       const void *B, const void *C, const float *D, float *y,
                       const float *h0, float *h_final,
                       int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                       int64_t ngroups, int64_t chunk_len, ssm_dtype_t in_dtype, uint32_t flags,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return ssd_fwd_call("ssd_chunk_scan_fwd", x, dt, dt_bias, A_log, B, C, D, y, h0, h_final, batch, L,
                        nheads, headdim, d_state, ngroups, chunk_len, in_dtype, flags, workspace,
                        workspace_bytes, stream, false);
}

int ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *dt_bias, const float *A_log,
                               const void *B, const void *C, const float *D, float *y,
                               const float *h0, float *h_final,
                               int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                               int64_t ngroups, int64_t chunk_len, ssm_dtype_t in_dtype, uint32_t flags,
                               hipStream_t stream) {
    return ssd_fwd_call("ssd_chunk_scan_fwd_noalloc", x, dt, dt_bias, A_log, B, C, D, y, h0, h_final, batch,
                        L, nheads, headdim, d_state, ngroups, chunk_len, in_dtype, flags, nullptr, 0, stream,
                        true);
}

size_t ssd_trap_chunk_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                              int64_t d_state, int64_t chunk_len) {
    (void)chunk_len;
    if (batch <= 0 || L <= 0 || nheads <= 0 || headdim <= 0 || d_state <= 0) return 0;
    return ssm::ssd_trap_workspace_bytes(batch, L, nheads, headdim, d_state);
}

int ssd_trap_chunk_scan_fwd(const void *x, const void *k, const void *q, const float *dt, const float *a,
                            const float *trap, const float *D, float *y, const float *h0,
                            const void *k_prev, const void *x_prev, float *h_final,
                            int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                            int64_t chunk_len, ssm_dtype_t in_dtype,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssd_trap_chunk_scan_fwd";
    REQUIRE_PTR(E, x); REQUIRE_PTR(E, k); REQUIRE_PTR(E, q); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, a);
    REQUIRE_PTR(E, trap); REQUIRE_PTR(E, y);
    int rc = ssd_check_shape(E, batch, L, nheads, headdim, d_state, nheads, chunk_len);
    if (rc != SSM_OK) return rc;
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if (in_dtype != SSM_BF16)
        return fail(SSM_ERR_UNSUPPORTED, "%s: the MFMA path takes bf16 x, k, q (SSM_BF16)", E);
    if ((k_prev == nullptr) != (x_prev == nullptr))
        return fail(SSM_ERR_INVALID_ARG, "%s: k_prev and x_prev must be given together", E);
    if (!(headdim == 32 || headdim == 64 || headdim == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: headdim %lld not in {32, 64, 128}", E, (long long)headdim);
    if (d_state % 32 != 0 || d_state > SSM_MAX_D_STATE)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld must be a multiple of 32 and <= %d", E,
                    (long long)d_state, SSM_MAX_D_STATE);
    if (!(chunk_len == 64 || chunk_len == 128 || chunk_len == 256))
        return fail(SSM_ERR_UNSUPPORTED, "%s: chunk_len %lld not in {64, 128, 256}", E, (long long)chunk_len);
    REQUIRE_ALIGN(E, x); REQUIRE_ALIGN(E, k); REQUIRE_ALIGN(E, q); REQUIRE_ALIGN(E, dt);
    REQUIRE_ALIGN(E, a); REQUIRE_ALIGN(E, trap); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, y);
    REQUIRE_ALIGN(E, h0); REQUIRE_ALIGN(E, k_prev); REQUIRE_ALIGN(E, x_prev); REQUIRE_ALIGN(E, h_final);
    REQUIRE_ALIGN(E, workspace);
    const void *ins[] = {x, k, q, dt, a, trap, k_prev, x_prev};
    for (size_t j = 0; j < sizeof(ins) / sizeof(ins[0]); ++j)
        if ((const void *)y == ins[j] || (h_final && (const void *)h_final == ins[j]))
            return fail(SSM_ERR_INVALID_ARG, "%s: an output aliases an input", E);
    const size_t need = ssm::ssd_trap_workspace_bytes(batch, L, nheads, headdim, d_state);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", E, need,
                    workspace ? workspace_bytes : (size_t)0);
    ssm::SsdTrapArgs args{x, k, q, dt, a, trap, D, y, h0, k_prev, x_prev, h_final,
                          batch, L, nheads, headdim, d_state, workspace};
    const char *kn = "ssd_trap";
    return launched(E, ssm::launch_ssd_trap(args, stream, &kn), kn);
}

size_t ssd_trap_rotate_qk_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t d_state,
                                         int64_t n_angles) {
    if (batch <= 0 || L <= 0 || nheads <= 0 || d_state <= 0 || n_angles < 0) return 0;
    return ssm::trap_rotate_workspace_bytes(batch, L, nheads, d_state, n_angles);
}

int ssd_trap_rotate_qk(const void *k_raw, const void *q_raw, const float *angles, const float *dt,
                       const float *angle_state, void *k, void *q, float *angle_state_out,
                       int64_t batch, int64_t L, int64_t nheads, int64_t d_state, int64_t n_angles,
                       ssm_dtype_t in_dtype, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssd_trap_rotate_qk";
    REQUIRE_PTR(E, k_raw); REQUIRE_PTR(E, q_raw); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, k); REQUIRE_PTR(E, q);
    REQUIRE_POS(E, batch); REQUIRE_POS(E, L); REQUIRE_POS(E, nheads); REQUIRE_POS(E, d_state);
    if (n_angles < 0)
        return fail(SSM_ERR_INVALID_ARG, "%s: n_angles must be >= 0 (got %lld)", E, (long long)n_angles);
    if (n_angles > 0) REQUIRE_PTR(E, angles);
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if (in_dtype != SSM_BF16)
        return fail(SSM_ERR_UNSUPPORTED, "%s: k and q are bf16 (SSM_BF16)", E);
    if (d_state % 2 != 0 || d_state > SSM_MAX_D_STATE)
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld must be even and <= %d", E, (long long)d_state,
                    SSM_MAX_D_STATE);
    if (2 * n_angles > d_state)
        return fail(SSM_ERR_INVALID_ARG, "%s: 2 * n_angles (%lld) exceeds d_state (%lld)", E,
                    (long long)(2 * n_angles), (long long)d_state);
    if (too_big(batch, L, nheads, d_state)) return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    REQUIRE_ALIGN(E, k_raw); REQUIRE_ALIGN(E, q_raw); REQUIRE_ALIGN(E, angles); REQUIRE_ALIGN(E, dt);
    REQUIRE_ALIGN(E, angle_state); REQUIRE_ALIGN(E, k); REQUIRE_ALIGN(E, q); REQUIRE_ALIGN(E, angle_state_out);
    REQUIRE_ALIGN(E, workspace);
    // k may be k_raw and q may be q_raw (rotated in place), and angle_state_out may
    // be angle_state; no other output may share memory with an input or output.
    {
        const void *so = angle_state_out;
        const void *others_k[] = {q, q_raw, angles, dt, angle_state, so};
        const void *others_q[] = {k, k_raw, angles, dt, angle_state, so};
        const void *others_s[] = {k_raw, q_raw, angles, dt, k, q};
        for (const void *o : others_k)
            if (o && o == k) return fail(SSM_ERR_INVALID_ARG, "%s: k aliases another argument", E);
        for (const void *o : others_q)
            if (o && o == q) return fail(SSM_ERR_INVALID_ARG, "%s: q aliases another argument", E);
        for (const void *o : others_s)
            if (so && o == so) return fail(SSM_ERR_INVALID_ARG, "%s: angle_state_out aliases another argument", E);
    }
    const size_t need = ssm::trap_rotate_workspace_bytes(batch, L, nheads, d_state, n_angles);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", E, need,
                    workspace ? workspace_bytes : (size_t)0);
    ssm::TrapRotArgs args{k_raw, q_raw, angles, dt, angle_state, k, q, angle_state_out,
                          batch, L, nheads, d_state, n_angles, workspace};
    const char *kn = "trap_rotate";
    return launched(E, ssm::launch_trap_rotate(args, stream, &kn), kn);
}

size_t ssd_trap_chunk_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                              int64_t d_state, int64_t chunk_len) {
    (void)chunk_len;
    if (batch <= 0 || L <= 0 || nheads <= 0 || headdim <= 0 || d_state <= 0) return 0;
    return ssm::ssd_trap_bwd_workspace_bytes(batch, L, nheads, headdim, d_state);
}

int ssd_trap_chunk_scan_bwd(const void *x, const void *k, const void *q, const float *dt, const float *a,
                            const float *trap, const float *D, const float *h0, const void *k_prev,
                            const void *x_prev, const float *dy, const float *dh_final,
                            float *dx, float *dk, float *dq, float *ddt, float *da, float *dtrap, float *dD,
                            float *dh0, float *dk_prev, float *dx_prev,
                            int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                            int64_t chunk_len, ssm_dtype_t in_dtype,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssd_trap_chunk_scan_bwd";
    REQUIRE_PTR(E, x); REQUIRE_PTR(E, k); REQUIRE_PTR(E, q); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, a);
    REQUIRE_PTR(E, trap); REQUIRE_PTR(E, dy);
    REQUIRE_PTR(E, dx); REQUIRE_PTR(E, dk); REQUIRE_PTR(E, dq); REQUIRE_PTR(E, ddt); REQUIRE_PTR(E, da);
    REQUIRE_PTR(E, dtrap);
    int rc = ssd_check_shape(E, batch, L, nheads, headdim, d_state, nheads, chunk_len);
    if (rc != SSM_OK) return rc;
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if (in_dtype != SSM_BF16)
        return fail(SSM_ERR_UNSUPPORTED, "%s: the MFMA path takes bf16 x, k, q (SSM_BF16)", E);
    if ((k_prev == nullptr) != (x_prev == nullptr))
        return fail(SSM_ERR_INVALID_ARG, "%s: k_prev and x_prev must be given together", E);
    if (!(headdim == 32 || headdim == 64 || headdim == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: headdim %lld not in {32, 64, 128}", E, (long long)headdim);
    if (!(d_state == 32 || d_state == 64 || d_state == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld not in {32, 64, 128}", E, (long long)d_state);
    if (!(chunk_len == 64 || chunk_len == 128 || chunk_len == 256))
        return fail(SSM_ERR_UNSUPPORTED, "%s: chunk_len %lld not in {64, 128, 256}", E, (long long)chunk_len);
    const void *ptrs[] = {x, k, q, dt, a, trap, D, h0, k_prev, x_prev, dy, dh_final, dx, dk, dq, ddt, da, dtrap,
                          dD, dh0, dk_prev, dx_prev, workspace};
    for (const void *pp : ptrs)
        if (!aligned16(pp)) return fail(SSM_ERR_UNSUPPORTED, "%s: a pointer is not 16-byte aligned", E);
    const void *ins[] = {x, k, q, dt, a, trap, D, h0, k_prev, x_prev, dy, dh_final};
    const void *outs[] = {dx, dk, dq, ddt, da, dtrap, dD, dh0, dk_prev, dx_prev};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        if (!outs[i]) continue;
        for (const void *in : ins)
            if (in == outs[i]) return fail(SSM_ERR_INVALID_ARG, "%s: an output aliases an input", E);
        for (size_t j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return fail(SSM_ERR_INVALID_ARG, "%s: two outputs alias", E);
    }
    const size_t need = ssm::ssd_trap_bwd_workspace_bytes(batch, L, nheads, headdim, d_state);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", E, need,
                    workspace ? workspace_bytes : (size_t)0);
    ssm::SsdTrapBwdArgs args{x, k, q, dt, a, trap, D, h0, k_prev, x_prev, dy, dh_final,
                             dx, dk, dq, ddt, da, dtrap, dD, dh0, dk_prev, dx_prev,
                             batch, L, nheads, headdim, d_state, workspace};
    const char *kn = "ssd_trap_bwd";
    return launched(E, ssm::launch_ssd_trap_bwd(args, stream, &kn), kn);
}

size_t ssd_chunk_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                         int64_t d_state, int64_t ngroups, int64_t chunk_len) {
    (void)ngroups; (void)chunk_len;
    if (batch <= 0 || L <= 0 || nheads <= 0 || headdim <= 0 || d_state <= 0) return 0;
    return ssm::ssd_bwd_workspace_bytes(batch, L, nheads, headdim, d_state, ngroups);
}

int ssd_chunk_scan_bwd(const void *x, const float *dt, const float *dt_bias, const float *A_log,
                       const void *B, const void *C, const float *D, const float *h0,
                       const float *dy, const float *dh_final,
                       float *dx, float *ddt, float *dB, float *dC, float *dA_log,
                       float *dD, float *ddt_bias, float *dh0,
                       int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                       int64_t ngroups, int64_t chunk_len, ssm_dtype_t in_dtype, uint32_t flags,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssd_chunk_scan_bwd";
    REQUIRE_PTR(E, x); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, dy);
    REQUIRE_PTR(E, dx); REQUIRE_PTR(E, ddt); REQUIRE_PTR(E, dB); REQUIRE_PTR(E, dC);
    REQUIRE_PTR(E, dA_log);
    int rc = ssd_check_shape(E, batch, L, nheads, headdim, d_state, ngroups, chunk_len);
    if (rc != SSM_OK) return rc;
    if (in_dtype != SSM_F32 && in_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARG, "%s: in_dtype %d is not SSM_F32 or SSM_BF16", E, (int)in_dtype);
    if (in_dtype != SSM_BF16)
        return fail(SSM_ERR_UNSUPPORTED, "%s: x, B, C must be bf16 (SSM_BF16)", E);
    if ((flags & ~0x3u) != 0 || (flags & 0x3u) == 0x3u)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x: only SSM_BBAR_ZOH/DT/ONE apply", E, flags);
    if (!(headdim == 32 || headdim == 64 || headdim == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: headdim %lld not in {32, 64, 128}", E, (long long)headdim);
    if (!(d_state == 32 || d_state == 64 || d_state == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: d_state %lld not in {32, 64, 128}", E, (long long)d_state);
    if (!(chunk_len == 64 || chunk_len == 128 || chunk_len == 256))
        return fail(SSM_ERR_UNSUPPORTED, "%s: chunk_len %lld not in {64, 128, 256}", E, (long long)chunk_len);
    if (batch * nheads * ((L + 31) / 32) > 0x7fffffffLL)
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    REQUIRE_ALIGN(E, x); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, h0);
    REQUIRE_ALIGN(E, dy); REQUIRE_ALIGN(E, dh_final);
    REQUIRE_ALIGN(E, dx); REQUIRE_ALIGN(E, ddt); REQUIRE_ALIGN(E, dB); REQUIRE_ALIGN(E, dC);
    REQUIRE_ALIGN(E, dA_log); REQUIRE_ALIGN(E, dD); REQUIRE_ALIGN(E, ddt_bias); REQUIRE_ALIGN(E, dh0);
    REQUIRE_ALIGN(E, workspace);
    const void *ins[] = {x, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, workspace};
    const void *outs[] = {dx, ddt, dB, dC, dA_log, dD, ddt_bias, dh0};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        if (outs[i] == nullptr) continue;
        for (size_t j = 0; j < sizeof(ins) / sizeof(ins[0]); ++j)
            if (outs[i] == ins[j]) return fail(SSM_ERR_INVALID_ARG, "%s: an output aliases an input", E);
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (outs[i] == outs[j]) return fail(SSM_ERR_INVALID_ARG, "%s: two outputs alias", E);
    }
    const size_t need = ssm::ssd_bwd_workspace_bytes(batch, L, nheads, headdim, d_state, ngroups);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", E, need,
                    workspace ? workspace_bytes : (size_t)0);
    ssm::SsdBwdArgs a{x, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final,
                      dx, ddt, dB, dC, dA_log, dD, ddt_bias, dh0,
                      batch, L, nheads, headdim, d_state, ngroups, flags, workspace};
    const char *kn = "ssd_bwd";
    return launched(E, ssm::launch_ssd_bwd(a, stream, &kn), kn);
}

size_t ssd_cplx_chunk_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t nheads,
                                              int64_t headdim, int64_t n_complex, int64_t ngroups,
                                              int64_t chunk_len) {
    (void)ngroups;
    if (batch <= 0 || L <= 0 || nheads <= 0 || headdim <= 0 || n_complex <= 0 || chunk_len <= 0) return 0;
    return ssm::cssd_workspace_bytes(batch, L, nheads, headdim, n_complex, chunk_len);
}

int ssd_cplx_chunk_scan_fwd(const float *x, const float *dt, const float *dt_bias,
                            const float *A_log, const float *B, const float *C, const float *D,
                            float *y, const float *h0, float *h_final,
                            int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                            int64_t n_complex, int64_t ngroups, int64_t chunk_len, uint32_t flags,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssd_cplx_chunk_scan_fwd";
    REQUIRE_PTR(E, x); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, y);
    int rc = ssd_check_shape(E, batch, L, nheads, headdim, n_complex, ngroups, chunk_len);
    if (rc != SSM_OK) return rc;
    if (ssm::cssd_prep_blocks(batch, L, nheads, ngroups) > 0x7fffffffLL)
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    if ((flags & ~0x1Fu) != 0 || (flags & 0x3u) == 0x3u || (flags & 0xCu) == 0xCu)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x not a valid combination", E, flags);
    if ((flags & 0xCu) == SSM_CPLX_CODE && (flags & 0x3u) != SSM_BBAR_ZOH)
        return fail(SSM_ERR_INVALID_ARG, "%s: SSM_CPLX_CODE fixes its own input scale; use SSM_BBAR_ZOH", E);
    if (!(headdim == 32 || headdim == 64 || headdim == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: headdim %lld not in {32, 64, 128}", E, (long long)headdim);
    if (n_complex % 8 != 0 || n_complex > 64)
        return fail(SSM_ERR_UNSUPPORTED, "%s: n_complex %lld must be a multiple of 8 and <= 64", E,
                    (long long)n_complex);
    if (!(chunk_len == 32 || chunk_len == 64 || chunk_len == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: chunk_len %lld not in {32, 64, 128}", E, (long long)chunk_len);
    REQUIRE_ALIGN(E, x); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, y);
    REQUIRE_ALIGN(E, h0); REQUIRE_ALIGN(E, h_final); REQUIRE_ALIGN(E, workspace);
    if ((const void *)y == (const void *)x || (const void *)y == (const void *)dt ||
        (const void *)y == (const void *)B || (const void *)y == (const void *)C)
        return fail(SSM_ERR_INVALID_ARG, "%s: y aliases an input", E);
    const size_t need = ssm::cssd_workspace_bytes(batch, L, nheads, headdim, n_complex, chunk_len);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", E, need,
                    workspace ? workspace_bytes : (size_t)0);
    ssm::CssdArgs a{x, dt, dt_bias, A_log, B, C, D, y, h0, h_final, batch, L, nheads, headdim,
                    n_complex, ngroups, chunk_len, flags, workspace};
    const char *kn = "cssd";
    return launched(E, ssm::launch_cssd(a, stream, &kn), kn);
}

size_t ssd_cplx_mimo_chunk_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t rank, int64_t nheads,
                                                   int64_t headdim, int64_t n_complex, int64_t ngroups,
                                                   int64_t chunk_len) {
    (void)ngroups;
    if (batch <= 0 || L <= 0 || rank <= 0 || nheads <= 0 || headdim <= 0 || n_complex <= 0 || chunk_len <= 0)
        return 0;
    return ssm::cssd_workspace_bytes(batch, L * rank, nheads, headdim, n_complex, chunk_len);
}

int ssd_cplx_mimo_chunk_scan_fwd(const float *x, const float *dt, const float *dt_bias,
                                 const float *A_log, const float *B, const float *C, const float *D,
                                 float *y, const float *h0, float *h_final,
                                 int64_t batch, int64_t L, int64_t rank, int64_t nheads, int64_t headdim,
                                 int64_t n_complex, int64_t ngroups, int64_t chunk_len, uint32_t flags,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *E = "ssd_cplx_mimo_chunk_scan_fwd";
    REQUIRE_PTR(E, x); REQUIRE_PTR(E, dt); REQUIRE_PTR(E, A_log); REQUIRE_PTR(E, B);
    REQUIRE_PTR(E, C); REQUIRE_PTR(E, y);
    if (!(rank == 1 || rank == 2 || rank == 4 || rank == 8 || rank == 16))
        return fail(SSM_ERR_UNSUPPORTED, "%s: rank %lld not in {1, 2, 4, 8, 16}", E, (long long)rank);
    REQUIRE_POS(E, L);
    if (L > (int64_t(1) << 40) / rank)
        return fail(SSM_ERR_UNSUPPORTED, "%s: L x rank too large", E);
    int rc = ssd_check_shape(E, batch, L * rank, nheads, headdim, n_complex, ngroups, chunk_len);   // rows
    if (rc != SSM_OK) return rc;
    if (ssm::cssd_prep_blocks(batch, L * rank, nheads, ngroups) > 0x7fffffffLL)
        return fail(SSM_ERR_UNSUPPORTED, "%s: problem too large", E);
    if ((flags & ~0x13u) != 0 || (flags & 0x3u) == 0x3u)
        return fail(SSM_ERR_INVALID_ARG, "%s: flags 0x%x not a valid combination (stable reading of A only)", E,
                    flags);
    if (!(headdim == 32 || headdim == 64 || headdim == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: headdim %lld not in {32, 64, 128}", E, (long long)headdim);
    if (n_complex % 8 != 0 || n_complex > 64)
        return fail(SSM_ERR_UNSUPPORTED, "%s: n_complex %lld must be a multiple of 8 and <= 64", E,
                    (long long)n_complex);
    if (!(chunk_len == 32 || chunk_len == 64 || chunk_len == 128))
        return fail(SSM_ERR_UNSUPPORTED, "%s: chunk_len %lld not in {32, 64, 128}", E, (long long)chunk_len);
    REQUIRE_ALIGN(E, x); REQUIRE_ALIGN(E, dt); REQUIRE_ALIGN(E, dt_bias); REQUIRE_ALIGN(E, A_log);
    REQUIRE_ALIGN(E, B); REQUIRE_ALIGN(E, C); REQUIRE_ALIGN(E, D); REQUIRE_ALIGN(E, y);
    REQUIRE_ALIGN(E, h0); REQUIRE_ALIGN(E, h_final); REQUIRE_ALIGN(E, workspace);
    if ((const void *)y == (const void *)x || (const void *)y == (const void *)dt ||
        (const void *)y == (const void *)B || (const void *)y == (const void *)C)
        return fail(SSM_ERR_INVALID_ARG, "%s: y aliases an input", E);
    const size_t need = ssm::cssd_workspace_bytes(batch, L * rank, nheads, headdim, n_complex, chunk_len);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", E, need,
                    workspace ? workspace_bytes : (size_t)0);
    ssm::CssdArgs a{x, dt, dt_bias, A_log, B, C, D, y, h0, h_final, batch, L, nheads, headdim,
                    n_complex, ngroups, chunk_len, flags, workspace, rank};
    const char *kn = "cssd";
    return launched(E, ssm::launch_cssd(a, stream, &kn), kn);
}

}  // extern "C"
