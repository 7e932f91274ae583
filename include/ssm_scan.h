/*
 * ssm_scan.h -- C interface of libssmscan.so, the MI355X (gfx950) selective
 * state-space scan library (forward scans and their gradients).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor is a caller-owned, contiguous, row-major device buffer on
 *    the current HIP device.  The library allocates and frees nothing and
 *    never synchronises; work is enqueued on `stream` and the call returns.
 *    A device fault therefore surfaces at the caller's next synchronisation.
 *  - Arguments are validated before any HIP call.  On a bad argument the
 *    function returns a negative ssm_status_t and nothing is launched;
 *    ssm_last_error() then holds "<entry point or kernel>: <reason>".
 *  - Optional inputs (dt_bias, D, h0) may be NULL, meaning zero.  h_final may
 *    be NULL (not written).  h0 == h_final is allowed (the state is carried
 *    in place); y must not alias any input.
 *  - All pointers must be 16-byte aligned (torch allocations are).
 *  - dt is the raw time step before softplus: delta = softplus(dt + dt_bias)
 *    is formed inside the kernels, exactly once.
 *  - Results are bitwise reproducible run to run (no floating-point atomics).
 *
 * Citations name the page and the section (source file and function) of the
 * prior art that defines each operation:
 *   [BF-S6]   @seanhogg/builderforce-memory-engine 2026.6.18,
 *             package/dist/kernels/selective_scan.js (header comment,
 *             softplus, discretise_A, discretise_B, forward_scan,
 *             forward_reduce)
 *   [BF-SSD]  same package, package/dist/kernels/ssd.js and ssd.d.ts
 *             (header comment, ssd_chunk_forward)
 *   [BF-CONV] same package, package/src/kernels/conv1d.ts (header comment,
 *             conv1d_forward)
 *   [BF-CSSD] same package, package/src/kernels/complex_ssd.ts (header
 *             comment, et_bbar_re/et_bbar_im, complex_ssd_forward)
 *   [BF-M3]   same package, package/src/model/mamba3_block.ts (module header
 *             item 2, the weight shapes, Mamba3BlockConfig.mimoGroup), and
 *             complex_ssd.ts header item 3
 *   [RS-M1]   mamba-rs 0.4.0, src/mamba_ssm/gpu/forward.rs
 *             (gpu_forward_mamba_layer, steps F4a, F4d and F4e, and GpuMambaDims)
 *   [RS-M3]   mamba-rs 0.2.1, src/mamba3_siso/gpu/mamba3_gpu.rs
 *             (module header; gpu_forward_mamba3_layer, steps F4e+f, F5,
 *             F5b and F6, kernels K2-K5 and the final-state writeback)
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of the large inputs (u or x, B, C); everything else is fp32 */
typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_INVALID_ARG = -1,  /* NULL required pointer, dim <= 0, H % G != 0, ... */
    SSM_ERR_UNSUPPORTED = -2,  /* a size or alignment outside what the kernels support */
    SSM_ERR_WORKSPACE = -3,    /* workspace missing or smaller than *_workspace_size() */
    SSM_ERR_HIP = -4           /* a launch failed; the message carries hipGetErrorString */
} ssm_status_t;

/* flags bit-field.
 * Bits 0-1 pick the input scale that multiplies B_t * u_t:
 *   SSM_BBAR_ZOH  exact zero-order hold, (exp(delta*A) - 1)/A  [BF-S6 discretise_B;
 *                 for A -> 0 it tends to delta]
 *   SSM_BBAR_DT   delta (the first-order limit of the hold)  [BF-S6 comment on
 *                 discretise; RS-M3 gamma = dt at trap = 1]
 *   SSM_BBAR_ONE  1 (B_t * x_t unscaled, as the SSD page kernel writes it) [BF-SSD]
 * Bits 2-3 pick how the complex entry point reads A_log[h] = [l, phi]:
 *   SSM_CPLX_STABLE  lambda = -exp(l) + i*phi  (decay times rotation; stable)
 *   SSM_CPLX_DOC     lambda = exp(l) * exp(i*phi)  (the page's header comment)
 *   SSM_CPLX_CODE    Abar = exp(delta*(l + i*phi)), beta = (Abar - 1)*exp(-l - i*phi)
 *                    (the page kernel taken literally)
 * Bit 4: SSM_CPLX_CONJ_C gives y = Re(conj(C).h) instead of Re(C.h). */
#define SSM_BBAR_ZOH    0x0u
#define SSM_BBAR_DT     0x1u
#define SSM_BBAR_ONE    0x2u
#define SSM_CPLX_STABLE 0x0u
#define SSM_CPLX_DOC    0x4u
#define SSM_CPLX_CODE   0x8u
#define SSM_CPLX_CONJ_C 0x10u

/* Largest state size any entry point accepts. */
#define SSM_MAX_D_STATE 256
/* Largest state size of the S6 scan with B, C per group of channels. */
#define SSM_MAX_D_STATE_GROUPED 32

/* Message of the last failing call made by this thread ("" if none). */
const char *ssm_last_error(void);

/* ------------------------------------------------------------------ S6 ----
 * Mamba-1 selective scan with a diagonal state per channel [BF-S6 header,
 * forward_scan, forward_reduce; RS-M1 F4d]:
 *   delta[b,t,d] = softplus(dt[b,t,d] + dt_bias[d])
 *   A[d,n]       = -exp(A_log[d,n])
 *   h_t[n]       = exp(delta*A[d,n]) * h_{t-1}[n] + beta(delta, A[d,n]) * B[b,t,n] * u[b,t,d]
 *   y[b,t,d]     = sum_n C[b,t,n] * h_t[n] + D[d] * u[b,t,d]
 * with h_{-1} = h0 (or 0) and h_final = h_{L-1}.  beta follows flags bits 0-1
 * (default SSM_BBAR_ZOH).  B and C are shared by all channels.
 *
 * Layouts: u (batch, L, d_inner) [in_dtype]; dt (batch, L, d_inner) fp32;
 * dt_bias, D (d_inner) fp32; A_log (d_inner, d_state) fp32;
 * B, C (batch, L, d_state) [in_dtype]; y (batch, L, d_inner) fp32;
 * h0, h_final (batch, d_inner, d_state) fp32.
 * Limits: 1 <= d_state <= 256; any L >= 1.
 *
 * Workspace (optional; caller-owned device memory, 16-byte aligned): for long
 * sequences over few channels (a quarter of the chip's blocks or fewer, L >=
 * 1024, d_state <= 16), ssm_s6_scan_fwd_workspace_size returns a nonzero size,
 * and a workspace of that size lets the call cut time into segments joined by
 * the associative carry of the recurrence ([BF-S6 forward_scan] tile carry,
 * with the earlier map applied first).  With workspace NULL the call walks the
 * sequence in one pass; both give the same result up to fp32 rounding order.
 * A non-NULL workspace smaller than the queried size is SSM_ERR_WORKSPACE.
 * The query returns 0 where the walk is used; workspace may then be NULL. */
size_t ssm_s6_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state);

int ssm_s6_scan_fwd(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                    const void *B, const void *C, const float *D, float *y,
                    const float *h0, float *h_final,
                    int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                    ssm_dtype_t in_dtype, uint32_t flags,
                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------- S6, B and C per channel group ----
 * The S6 scan above with B and C per group of channels instead of shared
 * [BF-S6 header: B and C are input-dependent; here they are also
 * per-channel]: channel d reads row g = d * ngroups / d_inner,
 *   h_t[n]   = exp(delta*A[d,n]) * h_{t-1}[n] + beta * B[b,t,g,n] * u[b,t,d]
 *   y[b,t,d] = sum_n C[b,t,g,n] * h_t[n] + D[d] * u[b,t,d].
 * ngroups = d_inner gives every channel its own B, C; ngroups = 1 is
 * ssm_s6_scan_fwd (and runs its kernel).
 *
 * Layouts: B, C (batch, L, ngroups, d_state) [in_dtype]; the rest as
 * ssm_s6_scan_fwd.  Limits: d_inner % ngroups == 0; d_state <= 32 when
 * ngroups > 1 (SSM_MAX_D_STATE_GROUPED; 256 at ngroups = 1).  No workspace. */
int ssm_s6_scan_grouped_fwd(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                            const void *B, const void *C, const float *D, float *y,
                            const float *h0, float *h_final,
                            int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                            ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream);

/* ------------------------------------------------ S6 with its layer ----
 * The Mamba-1 layer's steps on either side of the scan, fused into it
 * [BF-CONV header and conv1d_forward; RS-M1 F4a (conv1d burn-in with fused
 * SiLU and a carried conv state), F4d, F4e (gating)]:
 *   u[b,t,d] = SiLU(conv_b[d] + sum_{k<d_conv} conv_w[d,k] * x[b,t-k,d]),
 *              x[b,t',d] for t' < 0 taken from conv_state[b,d,d_conv-1+t'] (or 0)
 *   y[b,t,d] = (S6 scan of u as in ssm_s6_scan_fwd, D u included) * SiLU(z[b,t,d])
 * with SiLU(v) = v / (1 + exp(-v)); without z the output is not gated.
 * conv_state_out[b,d,j] = x at time L-(d_conv-1)+j (the old state's tail when
 * L < d_conv-1): what the next call carries.  One call with L = 1, with
 * h_final == h0 and conv_state_out == conv_state, is one decode step.
 *
 * Layouts: x, z (batch, L, d_inner) [in_dtype]; conv_w (d_inner, d_conv) fp32
 * (tap k multiplies x[t-k]); conv_b (d_inner) fp32 or NULL; conv_state,
 * conv_state_out (batch, d_inner, d_conv-1) fp32, oldest step first, or NULL;
 * u_out (batch, L, d_inner) fp32 or NULL (the scan's input, for a backward);
 * the rest as ssm_s6_scan_fwd.  h_final may be h0 and conv_state_out may be
 * conv_state; no other output may alias an input or another output.
 * Limits: 1 <= d_conv <= SSM_MAX_D_CONV; the rest as ssm_s6_scan_fwd.  No
 * workspace.  Arithmetic: fp32 (conv, SiLU and gate in the scan kernel). */
#define SSM_MAX_D_CONV 4

int ssm_s6_fused_fwd(const void *x, const float *conv_w, const float *conv_b, const float *conv_state,
                     const void *z, const float *dt, const float *dt_bias, const float *A_log,
                     const void *B, const void *C, const float *D, float *y,
                     const float *h0, float *h_final, float *u_out, float *conv_state_out,
                     int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t d_conv,
                     ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream);

/* ---------------------------------------------- causal conv1d alone ----
 * The causal depthwise convolution before a scan, on its own [BF-CONV header
 * and conv1d_forward; RS-M1 F4a for the fused SiLU and the carried state],
 * e.g. Mamba-2's convolution over the concatenated x, B, C channels:
 *   y[b,t,c] = bias[c] + sum_{k<d_conv} w[c,k] * x[b,t-k,c],
 *              x[b,t',c] for t' < 0 from state_in[b,c,d_conv-1+t'] (or 0),
 * followed by SiLU(v) = v / (1 + exp(-v)) when silu == 1.
 * state_out[b,c,j] = x at time L-(d_conv-1)+j (the old state's tail when
 * L < d_conv-1).
 * Layouts: x, y (batch, L, channels) [dtype] (y rounded to bf16 once when
 * dtype is SSM_BF16); w (channels, d_conv) fp32 (tap k multiplies x[t-k]);
 * bias (channels) fp32 or NULL; state_in, state_out (batch, channels,
 * d_conv-1) fp32, oldest step first, or NULL.  state_out may be state_in; y
 * may not alias any input (later steps re-read earlier inputs).
 * Limits: 1 <= d_conv <= SSM_MAX_D_CONV.  No workspace.  fp32 arithmetic. */
int ssm_causal_conv1d_fwd(const void *x, const float *w, const float *bias, const float *state_in, void *y,
                          float *state_out, int64_t batch, int64_t L, int64_t channels, int64_t d_conv,
                          int silu, ssm_dtype_t dtype, hipStream_t stream);

/* --------------------------------------------------------- S6 backward ----
 * Gradients of a scalar loss through the S6 scan above, given dy = dL/dy and
 * optionally dh_final = dL/dh_final: the reverse-time chain rule of the
 * recurrence [BF-S6 backward_scan, completed with beta's dependence on A and
 * the sums over channels for the shared B and C].  With g_t = dL/dh_t
 * (g_{L-1} = C_{L-1} dy_{L-1} + dh_final, g_t = C_t dy_t + exp(delta_{t+1} A) g_{t+1}):
 *   du[b,t,d]   = D[d] dy + sum_n g_t beta_t B[b,t,n]
 *   ddt[b,t,d]  = sigmoid(dt + dt_bias) * sum_n g_t (h_{t-1} A Abar_t + B u dbeta/ddelta)
 *   dB[b,t,n]   = sum_d g_t beta_t u[b,t,d]         dC[b,t,n] = sum_d dy[b,t,d] h_t[n]
 *   dA_log[d,n] = A sum_{b,t} g_t (h_{t-1} delta Abar_t + B u dbeta/dA)
 *   dD[d] = sum_{b,t} dy u,   ddt_bias[d] = sum_{b,t} ddt,   dh0 = g_0 Abar_0
 * (dbeta/ddelta, dbeta/dA = Abar, delta^2 phi1'(delta A) for SSM_BBAR_ZOH;
 * 1, 0 for SSM_BBAR_DT; 0, 0 for SSM_BBAR_ONE.)
 *
 * Inputs: those of ssm_s6_scan_fwd (same layouts, in_dtype and flags), plus
 * dy (batch, L, d_inner) fp32 and dh_final (batch, d_inner, d_state) fp32 or NULL.
 * Outputs (fp32, caller-owned, fully overwritten): du, ddt (batch, L, d_inner);
 * dB, dC (batch, L, d_state); dA_log (d_inner, d_state); dD, ddt_bias (d_inner);
 * dh0 (batch, d_inner, d_state).  dD, ddt_bias and dh0 may be NULL (not
 * written); the others are required.  No output may alias an input or
 * another output.
 * Limits: 1 <= d_state <= 16; 1 <= L < 2^31 - 16; d_inner < 2^25.
 * Workspace: ssm_s6_scan_bwd_workspace_size() bytes, 16-byte aligned, owned by
 * the caller and reused freely between calls on one stream: the state entering
 * every 16-step tile (batch * ceil(L/16) * d_inner * d_state fp32) and
 * per-block partial sums, added in a fixed order by a second kernel. */
#define SSM_S6_BWD_MAX_D_STATE 16

size_t ssm_s6_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state);

int ssm_s6_scan_bwd(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                    const void *B, const void *C, const float *D, const float *h0,
                    const float *dy, const float *dh_final,
                    float *du, float *ddt, float *dB, float *dC, float *dA_log,
                    float *dD, float *ddt_bias, float *dh0,
                    int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                    ssm_dtype_t in_dtype, uint32_t flags,
                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------- S6 backward, B and C per channel group ----
 * The backward of ssm_s6_scan_grouped_fwd: the chain rule of ssm_s6_scan_bwd
 * with B, C read per group of channels (channel d: row d * ngroups / d_inner),
 * and dB, dC (batch, L, ngroups, d_state) summed over each group's channels
 * (per channel when ngroups = d_inner) [BF-S6 backward_scan, per channel].
 * ngroups = 1 is ssm_s6_scan_bwd (and runs its kernels).
 *
 * Inputs, outputs and limits as ssm_s6_scan_bwd, with B, C, dB, dC of shape
 * (batch, L, ngroups, d_state), d_inner % ngroups == 0 and, when ngroups > 1,
 * d_inner * d_state < 2^26.
 * Workspace: ssm_s6_scan_grouped_bwd_workspace_size() bytes, 16-byte aligned,
 * caller-owned: the state entering every 16-step tile, per-batch-row partial
 * sums and, when a group holds several channels, per-channel dB, dC shares
 * (batch * L * d_inner * d_state fp32 each). */
size_t ssm_s6_scan_grouped_bwd_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                              int64_t ngroups);

int ssm_s6_scan_grouped_bwd(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                            const void *B, const void *C, const float *D, const float *h0,
                            const float *dy, const float *dh_final,
                            float *du, float *ddt, float *dB, float *dC, float *dA_log,
                            float *dD, float *ddt_bias, float *dh0,
                            int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                            ssm_dtype_t in_dtype, uint32_t flags,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------- S6 with saved states ----
 * The saved-state form of the pair above, for training: the backward needs
 * the state entering each 16-step tile, and either recomputes it in a first
 * pass (ssm_s6_scan_bwd) or reads what the forward saved (the backward's
 * need for saved or recomputed states: [BF-S6 backward_scan]).
 *
 * ssm_s6_scan_fwd_save is ssm_s6_scan_fwd (same inputs, outputs, layouts and
 * result, bit for bit when L > 1; at L = 1 the plain entry point runs its
 * one-step kernel, whose rounding differs) that also writes checkpoints (batch, ceil(L/16), d_inner, d_state)
 * fp32: entry [b, k, d, n] is the state h_{16k-1}[n] of channel d (h0, or 0,
 * at k = 0).  checkpoints is caller-owned, ssm_s6_scan_checkpoint_size()
 * bytes, 16-byte aligned, and aliases no other argument.  Limits: d_state <=
 * SSM_S6_BWD_MAX_D_STATE.
 *
 * ssm_s6_scan_bwd_saved is ssm_s6_scan_bwd given those checkpoints (read
 * only; the caller passes the same u, dt, dt_bias, A_log, B, h0 and flags as
 * to the forward that wrote them): it skips the recomputing pass.  Same
 * outputs, limits and workspace size as ssm_s6_scan_bwd (its checkpoint
 * region is left unused). */
size_t ssm_s6_scan_checkpoint_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state);

int ssm_s6_scan_fwd_save(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                         const void *B, const void *C, const float *D, float *y,
                         const float *h0, float *h_final, float *checkpoints,
                         int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                         ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream);

int ssm_s6_scan_bwd_saved(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                          const void *B, const void *C, const float *D, const float *h0,
                          const float *dy, const float *dh_final, const float *checkpoints,
                          float *du, float *ddt, float *dB, float *dC, float *dA_log,
                          float *dD, float *ddt_bias, float *dh0,
                          int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                          ssm_dtype_t in_dtype, uint32_t flags,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The same pair for S6 with B, C per group of channels (the inputs and
 * outputs of ssm_s6_scan_grouped_fwd / ssm_s6_scan_grouped_bwd, d_inner a
 * multiple of ngroups), for the same training use: the forward also writes
 * checkpoints in the layout above, and the backward reads them instead of
 * recomputing the states.  ngroups = 1 is the pair above.  Limits: d_state <=
 * SSM_S6_BWD_MAX_D_STATE; the backward's workspace is
 * ssm_s6_scan_grouped_bwd_workspace_size() (its checkpoint region unused). */
int ssm_s6_scan_grouped_fwd_save(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                                 const void *B, const void *C, const float *D, float *y,
                                 const float *h0, float *h_final, float *checkpoints,
                                 int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                                 ssm_dtype_t in_dtype, uint32_t flags, hipStream_t stream);

int ssm_s6_scan_grouped_bwd_saved(const void *u, const float *dt, const float *dt_bias, const float *A_log,
                                  const void *B, const void *C, const float *D, const float *h0,
                                  const float *dy, const float *dh_final, const float *checkpoints,
                                  float *du, float *ddt, float *dB, float *dC, float *dA_log,
                                  float *dD, float *ddt_bias, float *dh0,
                                  int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                                  ssm_dtype_t in_dtype, uint32_t flags,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ----------------------------------------------------------------- SSD ----
 * Mamba-2 state-space dual scan with a scalar A per head [BF-SSD header and
 * ssd_chunk_forward; RS-M3 F6 K2-K5]:
 *   delta[b,t,h] = softplus(dt[b,t,h] + dt_bias[h]),  a = delta * A_h,  A_h = -exp(A_log[h])
 *   S_t[p,n]     = exp(a) * S_{t-1}[p,n] + sigma_t * x[b,t,h,p] * B[b,t,g,n]
 *   y[b,t,h,p]   = sum_n C[b,t,g,n] * S_t[p,n] + D[h] * x[b,t,h,p]
 * with group g = floor(h * ngroups / nheads), S_{-1} = h0 (or 0) and
 * h_final = S_{L-1}.  sigma follows flags bits 0-1 (default SSM_BBAR_DT,
 * i.e. sigma = delta).  The method cuts the sequence into chunks; the result
 * does not depend on the chunk length beyond rounding.  chunk_len is checked
 * against the limits below and otherwise only names the caller's model
 * setting: the kernels walk the sequence in their own 32-step chunks, carrying
 * the state on chip from chunk to chunk.  A long sequence is first cut into a
 * few segments whose own final states and entering states go through the
 * workspace, so that many (batch, segment, head) groups run at once.
 *
 * Layouts: x (batch, L, nheads, headdim) bf16; dt (batch, L, nheads) fp32;
 * dt_bias, A_log, D (nheads) fp32; B, C (batch, L, ngroups, d_state) bf16;
 * y (batch, L, nheads, headdim) fp32; h0, h_final (batch, nheads, headdim, d_state) fp32.
 * in_dtype must be SSM_BF16 (the contractions run on bf16 MFMA; SSM_F32 returns
 * SSM_ERR_UNSUPPORTED).  Limits: nheads % ngroups == 0; headdim in {32, 64, 128};
 * nheads * headdim <= 2^24 (as for every SSD-family call below); d_state a
 * multiple of 32, <= 256; chunk_len in {64, 128, 256}.
 * Workspace: ssd_chunk_scan_fwd_workspace_size() bytes, 16-byte aligned,
 * owned by the caller and reused freely between calls on one stream (one fp32
 * headdim x d_state state and one decay per (batch, head, segment)); the size
 * is a function of the shape only, and 0 when the sequence is one segment
 * (workspace may then be NULL). */
size_t ssd_chunk_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                         int64_t d_state, int64_t ngroups, int64_t chunk_len);

int ssd_chunk_scan_fwd(const void *x, const float *dt, const float *dt_bias, const float *A_log,
                       const void *B, const void *C, const float *D, float *y,
                       const float *h0, float *h_final,
                       int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                       int64_t ngroups, int64_t chunk_len, ssm_dtype_t in_dtype, uint32_t flags,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ssd_chunk_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace: the segment states go to the library's static device
 * scratch, SSM_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held by each GPU the
 * library runs on until the process ends; its address on a device is looked up
 * on the first call there.  The call allocates and frees nothing.
 * Arguments, layouts, limits and results are those of ssd_chunk_scan_fwd (the
 * same kernels, bit for bit), plus: a shape whose segment states need more than
 * the scratch (ssd_chunk_scan_fwd_workspace_size() > SSM_NOALLOC_SCRATCH_BYTES)
 * returns SSM_ERR_WORKSPACE before any HIP call.  Every call on one GPU shares
 * that GPU's scratch: calls that overlap on one GPU (concurrent streams, or
 * threads) race on it and must be serialised by the caller.  Nothing in the
 * scratch needs to start at zero (each call writes every slot it reads). */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *dt_bias, const float *A_log,
                               const void *B, const void *C, const float *D, float *y,
                               const float *h0, float *h_final,
                               int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                               int64_t ngroups, int64_t chunk_len, ssm_dtype_t in_dtype, uint32_t flags,
                               hipStream_t stream);

/* -------------------------------------------------------- SSD backward ----
 * Gradients of a scalar loss through the SSD scan above, given dy = dL/dy and
 * optionally dh_final = dL/dh_final: the reverse-time chain rule of the
 * recurrence [BF-SSD ssd_chunk_forward; the page's per-chunk backward,
 * ssd_chunk_backward, completed with the carry from later chunks].  With
 * G_t = dL/dS_t (G_{L-1} = dh_final + dy_{L-1} (x) C_{L-1}, G_t = e^{a_{t+1}} G_{t+1} + dy_t (x) C_t):
 *   dx[b,t,h,p] = D[h] dy + sigma_t sum_n G_t[p,n] B[b,t,g,n]
 *   dB[b,t,g,n] = sum over the group's heads of sigma_t sum_p x[b,t,h,p] G_t[p,n]
 *   dC[b,t,g,n] = sum over the group's heads of sum_p dy[b,t,h,p] S_t[p,n]
 *   ddt[b,t,h]  = sigmoid(dt + dt_bias) (da_t A + dsigma_t dsigma/ddelta),
 *                 da_t = e^{a_t} sum_{p,n} G_t S_{t-1},  dsigma_t = sum_{p,n} G_t x_t[p] B_t[n]
 *   dA_log[h]   = A sum_{b,t} (da_t delta_t + dsigma_t dsigma/dA)
 *   dD[h] = sum dy x,   ddt_bias[h] = sum ddt,   dh0 = e^{a_0} G_0
 *
 * Inputs: those of ssd_chunk_scan_fwd (same layouts, bf16 x, B, C; flags as
 * there), plus dy (batch, L, nheads, headdim) fp32 and dh_final
 * (batch, nheads, headdim, d_state) fp32 or NULL.
 * Outputs (fp32, caller-owned, fully overwritten): dx (batch, L, nheads, headdim);
 * ddt (batch, L, nheads); dB, dC (batch, L, ngroups, d_state); dA_log, dD,
 * ddt_bias (nheads); dh0 (batch, nheads, headdim, d_state).  dD, ddt_bias and
 * dh0 may be NULL (not written); the others are required.  No output may
 * alias an input or another output.
 * Limits: nheads % ngroups == 0; headdim in {32, 64, 128}; d_state in
 * {32, 64, 128}; chunk_len in {64, 128, 256} (checked; the kernels use their
 * own 32-step chunks).  in_dtype must be SSM_BF16.
 * Workspace: ssd_chunk_scan_bwd_workspace_size() bytes, 16-byte aligned, owned
 * by the caller: segment states in both directions, each head's share of dB
 * and dC (2 * batch * L * nheads * d_state fp32) and per-step scalars. */
size_t ssd_chunk_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                         int64_t d_state, int64_t ngroups, int64_t chunk_len);

int ssd_chunk_scan_bwd(const void *x, const float *dt, const float *dt_bias, const float *A_log,
                       const void *B, const void *C, const float *D, const float *h0,
                       const float *dy, const float *dh_final,
                       float *dx, float *ddt, float *dB, float *dC, float *dA_log,
                       float *dD, float *ddt_bias, float *dh0,
                       int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                       int64_t ngroups, int64_t chunk_len, ssm_dtype_t in_dtype, uint32_t flags,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------ trapezoidal SSD ----
 * Mamba-3 SISO recurrence with the trapezoidal input rule, per-step decay and
 * per-head k, q [RS-M3 module header, F5b m3_compute_abg, F6 and its carried
 * ssm / k / v states]:
 *   alpha_t = exp(a[b,t,h] * dt[b,t,h]),  beta_t = alpha_t dt_t (1 - trap_t),  gamma_t = trap_t dt_t
 *   S_t[p,n] = alpha_t S_{t-1}[p,n] + beta_t x_{t-1}[p] k_{t-1}[n] + gamma_t x_t[p] k_t[n]
 *   y[b,t,h,p] = sum_n q[b,t,h,n] S_t[p,n] + D[h] x[b,t,h,p]
 * with S_{-1} = h0 (or 0), (x_{-1}, k_{-1}) = (x_prev, k_prev) (or 0) and
 * h_final = S_{L-1}.  dt is the step as the model hands it over (already
 * positive: no softplus or bias is applied here), a the per-step decay rate
 * (a <= 0 for a contracting state) and trap the per-step blend in [0, 1]
 * (1 gives the plain SSD scan with sigma = dt).  The data-dependent rotation
 * of k and q is applied by the caller before this call.  A caller that cuts a
 * sequence into pieces passes each piece's h_final and its last x and k as the
 * next piece's h0, x_prev and k_prev.
 * The kernels run the SSD chunked scan on the shifted state
 * S'_t = S_t + dt_{t+1} (1 - trap_{t+1}) x_t (x) k_t, which follows the SSD
 * recurrence with input scale gamma_t + dt_{t+1} (1 - trap_{t+1}) (gamma only at
 * the last step) while the diagonal of each chunk uses gamma_t.
 *
 * Layouts: x (batch, L, nheads, headdim) bf16; k, q (batch, L, nheads, d_state)
 * bf16; dt, a, trap (batch, L, nheads) fp32; D (nheads) fp32 or NULL;
 * y (batch, L, nheads, headdim) fp32; h0, h_final (batch, nheads, headdim,
 * d_state) fp32 or NULL; x_prev (batch, nheads, headdim) and k_prev
 * (batch, nheads, d_state) bf16, both given or both NULL.  No output may
 * alias an input; h0 == h_final is allowed.
 * Limits: in_dtype SSM_BF16; headdim in {32, 64, 128}; d_state a multiple of
 * 32, <= 256; chunk_len in {64, 128, 256} (checked; the kernels use their own
 * 32-step chunks).
 * Workspace: ssd_trap_chunk_scan_fwd_workspace_size() bytes, 16-byte aligned,
 * owned by the caller, always required (segment states and decays as for
 * ssd_chunk_scan_fwd, plus the entering state with the carried input folded
 * in). */
size_t ssd_trap_chunk_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                              int64_t d_state, int64_t chunk_len);

int ssd_trap_chunk_scan_fwd(const void *x, const void *k, const void *q, const float *dt, const float *a,
                            const float *trap, const float *D, float *y, const float *h0,
                            const void *k_prev, const void *x_prev, float *h_final,
                            int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                            int64_t chunk_len, ssm_dtype_t in_dtype,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------- trapezoidal SSD backward ----
 * Gradients of a scalar loss through ssd_trap_chunk_scan_fwd, given dy and
 * optionally dh_final: the reverse-time chain rule of the trapezoidal
 * recurrence [RS-M3 module header, F5b, F6 and its chunked backward].  With
 * G_t = dL/dS_t (G_{L-1} = dh_final + dy_{L-1} (x) q_{L-1}, G_t = dy_t (x) q_t + alpha_{t+1} G_{t+1}):
 *   dq_t = S_t^T dy_t,   dx_t = D dy_t + gamma_t G_t k_t + beta_{t+1} G_{t+1} k_t,
 *   dk_t = gamma_t G_t^T x_t + beta_{t+1} G_{t+1}^T x_t   (the step before 0: x_prev, k_prev)
 *   dalpha_t = <G_t, S_{t-1}>, dbeta_t = <G_t, x_{t-1} (x) k_{t-1}>, dgamma_t = <G_t, x_t (x) k_t>
 *   da_t = dt_t (dalpha_t alpha_t + dbeta_t beta_t)
 *   ddt_t = dalpha_t a_t alpha_t + dbeta_t (1 - trap_t) alpha_t (1 + a_t dt_t) + dgamma_t trap_t
 *   dtrap_t = (dgamma_t - dbeta_t alpha_t) dt_t,  dD = sum dy x,  dh0 = alpha_0 G_0.
 * The kernels run the SSD backward of the shifted state (input scale
 * sigma_t = gamma_t + dt_{t+1}(1 - trap_{t+1}), k as B, q as C), add the
 * gradient of each chunk diagonal's gamma in place of sigma, and chain the
 * per-step gradients to dt, a and trap.
 *
 * Inputs: those of ssd_trap_chunk_scan_fwd (same layouts), dy (batch, L,
 * nheads, headdim) fp32 and dh_final (batch, nheads, headdim, d_state) fp32 or
 * NULL.  Outputs (fp32, caller-owned, fully overwritten): dx (batch, L,
 * nheads, headdim); dk, dq (batch, L, nheads, d_state); ddt, da, dtrap (batch,
 * L, nheads); dD (nheads) or NULL; dh0 (batch, nheads, headdim, d_state) or
 * NULL; dk_prev (batch, nheads, d_state), dx_prev (batch, nheads, headdim) or
 * NULL (written when the carried pair is given).  No output may alias an input
 * or another output.
 * Limits: in_dtype SSM_BF16; headdim and d_state in {32, 64, 128}; chunk_len in
 * {64, 128, 256} (checked; the kernels use their own 32-step chunks).
 * Workspace: ssd_trap_chunk_scan_bwd_workspace_size() bytes, 16-byte aligned,
 * owned by the caller (the SSD backward's scratch without per-head shares, the
 * entering state with the carried input folded in, its gradient, and one float
 * per (b, t, h) for the diagonal's gradient). */
size_t ssd_trap_chunk_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                                              int64_t d_state, int64_t chunk_len);

int ssd_trap_chunk_scan_bwd(const void *x, const void *k, const void *q, const float *dt, const float *a,
                            const float *trap, const float *D, const float *h0, const void *k_prev,
                            const void *x_prev, const float *dy, const float *dh_final,
                            float *dx, float *dk, float *dq, float *ddt, float *da, float *dtrap, float *dD,
                            float *dh0, float *dk_prev, float *dx_prev,
                            int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                            int64_t chunk_len, ssm_dtype_t in_dtype,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------- Mamba-3 k, q rotation ----
 * Data-dependent rotation of k and q ahead of ssd_trap_chunk_scan_fwd [RS-M3
 * F5 m3_angle_dt_fwd_seq (angle * dt accumulated per step, carried in the
 * layer's angle state) and F4e+f rope_fwd (k and q turned by the accumulated
 * angles)].  Per (b, h) and angle j < n_angles:
 *   theta_t[j] = angle_state[b,h,j] + sum_{s<=t} angles[b,s,j] * dt[b,s,h]
 *   (k[2j], k[2j+1]) = (kr[2j] cos theta - kr[2j+1] sin theta, kr[2j] sin theta + kr[2j+1] cos theta)
 * and the same for q; pairs j >= n_angles are copied unchanged, and
 * angle_state_out[b,h,j] = theta_{L-1}[j].  The page shows these launches but
 * not their bodies: the pairing (2j, 2j+1) and the direction of the turn are
 * the reading under which a rotated scan with trap = 1 is the complex-diagonal
 * SSD with lambda = -exp(l) + i phi for angles = -phi.
 * Arithmetic is fp32 (the angle is accumulated per segment of the sequence,
 * then step by step), the outputs are rounded once to bf16.
 *
 * Layouts: k_raw, q_raw, k, q (batch, L, nheads, d_state) bf16; angles
 * (batch, L, n_angles) fp32, shared by the heads; dt (batch, L, nheads) fp32
 * (as given to the scan); angle_state, angle_state_out (batch, nheads,
 * n_angles) fp32 or NULL (zero / not written).  k may be k_raw and q may be
 * q_raw (in place); angle_state_out may be angle_state; no other aliasing.
 * Limits: in_dtype SSM_BF16; d_state even, <= 256; 0 <= n_angles <= d_state/2
 * (0 copies k and q; angles may then be NULL).
 * Workspace: ssd_trap_rotate_qk_workspace_size() bytes, 16-byte aligned, owned
 * by the caller (one fp32 angle sum per (batch, segment, head, angle) and a
 * copy of the entering angle state). */
size_t ssd_trap_rotate_qk_workspace_size(int64_t batch, int64_t L, int64_t nheads, int64_t d_state,
                                         int64_t n_angles);

int ssd_trap_rotate_qk(const void *k_raw, const void *q_raw, const float *angles, const float *dt,
                       const float *angle_state, void *k, void *q, float *angle_state_out,
                       int64_t batch, int64_t L, int64_t nheads, int64_t d_state, int64_t n_angles,
                       ssm_dtype_t in_dtype, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------- complex SSD ----
 * Mamba-3-style SSD with a complex diagonal state [BF-CSSD header,
 * et_bbar_re/et_bbar_im, complex_ssd_forward]:
 *   lambda_h from A_log[h] = [l, phi] per flags bits 2-3 (default STABLE)
 *   Abar_t   = exp(delta_t * lambda_h),  beta_t = (Abar_t - 1)/lambda_h  (exact ET)
 *   h_t[p,n] = Abar_t * h_{t-1}[p,n] + beta_t * B[b,t,g,n] * x[b,t,h,p]   (complex)
 *   y[b,t,h,p] = Re(sum_n C[b,t,g,n] * h_t[p,n]) + D[h] * x[b,t,h,p]
 * flags bits 0-1 may replace beta by delta (DT) or 1 (ONE); SSM_CPLX_CONJ_C
 * uses conj(C).
 *
 * Layouts (all fp32): x (batch, L, nheads, headdim); dt (batch, L, nheads);
 * dt_bias, D (nheads); A_log (nheads, 2); B, C (batch, L, ngroups, n_complex, 2)
 * interleaved (re, im); y (batch, L, nheads, headdim);
 * h0, h_final (batch, nheads, headdim, n_complex, 2).
 * Limits: nheads % ngroups == 0; headdim in {32, 64, 128}; n_complex a
 * multiple of 8, <= 64; chunk_len in {32, 64, 128} (checked; the kernels use
 * their own 32-step chunks, and the result does not depend on it beyond
 * rounding).  Contractions run in fp32 on the matrix cores.
 * Workspace: ssd_cplx_chunk_scan_fwd_workspace_size() bytes (never 0),
 * 16-byte aligned, owned by the caller: per (batch, head, 32-step chunk) a
 * 528-byte record of the chunk's decays and input scales and the 3 KiB of
 * its decay-masked C.B^T tiles, and, when the sequence is cut into segments,
 * one complex headdim x n_complex state and one complex decay per (batch,
 * head, segment).  NULL or too small: SSM_ERR_WORKSPACE, nothing launched. */
size_t ssd_cplx_chunk_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t nheads,
                                              int64_t headdim, int64_t n_complex, int64_t ngroups,
                                              int64_t chunk_len);

int ssd_cplx_chunk_scan_fwd(const float *x, const float *dt, const float *dt_bias,
                            const float *A_log, const float *B, const float *C, const float *D,
                            float *y, const float *h0, float *h_final,
                            int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                            int64_t n_complex, int64_t ngroups, int64_t chunk_len, uint32_t flags,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------ complex SSD, multi-input multi-output ----
 * The MIMO form of the complex SSD [BF-M3]: per head, R = rank input vectors
 * and R outputs per step share one complex state (G x G blocks per head, with
 * B and C widened to R sets of n_complex entries).  The pages describe it and
 * leave it unimplemented; read as:
 *   h_t[p,n]     = Abar_t * h_{t-1}[p,n] + beta_t * sum_r B[b,t,r,g,n] * x[b,t,r,h,p]
 *   y[b,t,r,h,p] = Re(sum_n C[b,t,r,g,n] * h_t[p,n]) + D[h] * x[b,t,r,h,p]
 * with Abar, beta, lambda as for ssd_cplx_chunk_scan_fwd (stable reading of A
 * only).  Every input of step t enters h_t before any output of step t is
 * read.  rank 1 is ssd_cplx_chunk_scan_fwd.
 *
 * Layouts (all fp32): x, y (batch, L, rank, nheads, headdim); dt (batch, L,
 * nheads); dt_bias, D (nheads); A_log (nheads, 2); B, C (batch, L, rank,
 * ngroups, n_complex, 2) interleaved (re, im); h0, h_final (batch, nheads,
 * headdim, n_complex, 2).
 * flags: SSM_BBAR_* and SSM_CPLX_CONJ_C (SSM_CPLX_DOC / SSM_CPLX_CODE are
 * rejected).  Limits: rank in {1, 2, 4, 8, 16}; otherwise as for
 * ssd_cplx_chunk_scan_fwd, with L x rank in place of L.
 * Workspace: ssd_cplx_mimo_chunk_scan_fwd_workspace_size() bytes, as for
 * ssd_cplx_chunk_scan_fwd over L x rank rows. */
size_t ssd_cplx_mimo_chunk_scan_fwd_workspace_size(int64_t batch, int64_t L, int64_t rank, int64_t nheads,
                                                   int64_t headdim, int64_t n_complex, int64_t ngroups,
                                                   int64_t chunk_len);

int ssd_cplx_mimo_chunk_scan_fwd(const float *x, const float *dt, const float *dt_bias,
                                 const float *A_log, const float *B, const float *C, const float *D,
                                 float *y, const float *h0, float *h_final,
                                 int64_t batch, int64_t L, int64_t rank, int64_t nheads, int64_t headdim,
                                 int64_t n_complex, int64_t ngroups, int64_t chunk_len, uint32_t flags,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */
