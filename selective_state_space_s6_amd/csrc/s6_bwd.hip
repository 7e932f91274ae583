// s6_bwd.hip -- backward pass of the S6 (Mamba-1) selective scan, gfx950.
//
// Gradients of a loss with respect to every input of the forward scan of
// s6_scan.hip, given dL/dy and optionally dL/dh_final: the reverse-time chain
// rule of the recurrence (the reverse scan of builderforce-memory-engine
// selective_scan.js, backward_scan, completed with beta's dependence on A and
// the sums over channels for the shared B and C):
//   g_t      = g_{t+1} Abar_{t+1} + C_t dy_t          (g after the last step = dL/dh_final)
//   dC_t[n]  = sum_d dy_t[d] h_t[d,n]
//   dB_t[n]  = sum_d g_t beta_t u_t[d]
//   du_t[d]  = D dy_t + sum_n g_t beta_t B_t[n]
//   ddt_t[d] = sigmoid(dt + dt_bias) sum_n g_t (h_{t-1} A Abar + B_t u_t dbeta/ddelta)
//   dA_log   = A sum_{b,t} g_t (h_{t-1} delta Abar + B_t u_t dbeta/dA)
//   dD = sum dy u,  ddt_bias = sum ddt,  dh0 = g_0 Abar_0
// For the zero-order hold beta = (Abar - 1)/A, dbeta/ddelta = Abar and
// dbeta/dA = (delta Abar - beta)/A (= delta^2 phi1'(delta A)); for beta = delta
// they are 1 and 0, for beta = 1 both are 0.
//
// s6_bwd_kernel: one 256-thread block per (batch row, 16 channels); lane
// (n, k) = (tid / 16, tid % 16) owns state n of channel d0 + k, so a 16-lane
// DPP row is 16 channels sharing one state (B[t, n], C[t, n] of a tile sit one
// step per lane and reach the row with row_newbcast) and a wave holds 4 states.
//   pass 1  forward over the sequence in 16-step tiles, storing the state that
//           enters each tile (checkpoints) -- skipped when the forward saved
//           them (ssm_s6_scan_fwd_save), the same layout read in place;
//   pass 2  backward over the tiles: recompute the tile's 16 states from its
//           checkpoint into registers, then run the adjoint.
// Global loads of the next tile are issued before a tile is computed; delta,
// u, dy are staged once per (t, d) through double-buffered LDS.
// Reductions: sums over states (du, ddt) first over the wave's 4 rows with
// permlane32/permlane16 swaps (4 values -> one register holding 4 sums), then
// over the 4 waves through LDS; sums over the block's 16 channels (dB, dC)
// through LDS (bank-swizzled rows read as 128-bit words) into per-block
// partials in the workspace.
// s6_bwd_reduce_kernel: adds the per-block partials of dB, dC over channel
// blocks and the per-batch-row partials of dA_log, dD, ddt_bias over the
// batch, in a fixed order (bitwise reproducible; no atomics).
#include "device_common.hpp"
#include "launchers.hpp"
#include <type_traits>
#include <utility>

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr int kT = 16;        // time steps per tile == lanes per DPP row
constexpr int kTS = kT + 4;   // padded LDS row of a staged (channel, 16 steps)
constexpr int kCW = 16;       // channels per block

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

struct S6BKp {
    const void *u; const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; const float *h0;
    const float *dy; const float *dhf;
    float *du, *ddt, *dB, *dC, *dA_log, *dD, *ddt_bias, *dh0;
    float *ck;            // (batch, ntiles, d_inner, N): state entering each tile
    bool saved;           // ck holds the forward's saved states: pass 1 is skipped
    float *pB, *pC;       // (ncblk, batch, L, N): per channel-block partials
    float *pA;            // (batch, d_inner, N): per batch-row partials of dA (not yet times A)
    float *pDv, *pTb;     // (batch, d_inner): per batch-row partials of dD, ddt_bias
    int64_t batch, L, Dm, N, ntiles, ncblk;
};

// phi1'(z) = sum_k k z^(k-1)/(k+1)! to z^3 (|z| < 1/8: truncation < 4e-6 relative)
__device__ __forceinline__ float dphi1_series(float z) {
    float q = fmaf(z, 1.0f / 30.0f, 1.0f / 8.0f);
    q = fmaf(z, q, 1.0f / 3.0f);
    return fmaf(z, q, 0.5f);
}

__device__ __forceinline__ float fadd_u(uint32_t a, uint32_t b) {
    return __uint_as_float(a) + __uint_as_float(b);
}
// Four per-lane values v0..v3 -> one register whose row rho holds the sum over
// the wave's 4 rows of v[perm(rho)], perm = (0, 2, 1, 3).
__device__ __forceinline__ float rows_reduce4(float v0, float v1, float v2, float v3) {
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
    const float z1 = fadd_u(s1[0], s1[1]);
    const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
    const float z2 = fadd_u(s2[0], s2[1]);
    const auto s3 = __builtin_amdgcn_permlane16_swap(__float_as_uint(z1), __float_as_uint(z2), false, false);
    return fadd_u(s3[0], s3[1]);
}

__device__ __forceinline__ int64_t ck_step_n(const S6BKp &p) { return p.Dm * p.N; }

struct StageRaw { float dt, u, dy; };    // staging role: (time tl, channel c) of one tile
struct LaneRaw { float B, C, hin; };     // lane role: B, C of step k, state n; entering state

struct Lds {
    float sDl[2][kCW][kTS];   // delta
    float sU[2][kCW][kTS];    // u
    float sDy[2][kCW][kTS];   // dy
    float sDD[4][2][kT][kCW]; // [wave][du, ddt][t][channel]
    float sBC[2][kT][16][16]; // [dB, dC][t][state][swizzled channel]
};

template <typename TIN, int MODE>
__device__ __forceinline__ void s6_bwd_body(const S6BKp &p, Lds &S) {
    auto &sDl = S.sDl;
    auto &sU = S.sU;
    auto &sDy = S.sDy;
    auto &sDD = S.sDD;
    auto &sBC = S.sBC;
    const int tid = threadIdx.x;
    const int n = tid >> 4, k = tid & 15;          // lane role: state, channel
    const int wv = tid >> 6, rho = (tid >> 4) & 3; // wave, row within the wave
    const int64_t work = xcd_swizzle(blockIdx.x, gridDim.x);
    const int64_t b = work / p.ncblk, cb = work % p.ncblk;
    const int64_t d0 = cb * kCW;
    const int64_t d = d0 + k;
    const bool ok = d < p.Dm && n < p.N;
    const int64_t dcn = min(d, p.Dm - 1), ncn = min((int64_t)n, p.N - 1);
    const int L = (int)p.L;                        // L < 2^31 (checked by the caller)
    const int ntiles = (int)p.ntiles;

    const float al = ok ? p.A_log[d * p.N + n] : 0.0f;
    const float A = ok ? -fminf(expf(al), kMaxAbsA) : 0.0f;
    const float A2 = A * kLog2e;
    const float iA = ok ? -expf(-al) : 0.0f;      // 1/A

    // staging role: thread (tl, c) handles time step tl of channel d0 + c
    const int tl = tid >> 4, c = tid & 15;
    const int64_t dcs = d0 + c;
    const bool cok = dcs < p.Dm;
    const int64_t dcl = min(dcs, p.Dm - 1);
    const float bias = (cok && p.dt_bias) ? p.dt_bias[dcs] : 0.0f;
    const float Dv = (cok && p.D) ? p.D[dcs] : 0.0f;

    // Addresses: a block-uniform base (scalar registers) per tile plus a 32-bit
    // per-lane byte offset (the lane's step within the tile times the row pitch,
    // plus its channel or state), which stays far below 4 GiB.  Steps past L
    // re-read step L - 1; their values are masked where they are consumed.
    const float *dt_b = p.dt + (b * p.L) * p.Dm + d0;
    const TIN *u_b = static_cast<const TIN *>(p.u) + (b * p.L) * p.Dm + d0;
    const float *dy_b = p.dy + (b * p.L) * p.Dm + d0;
    float *du_b = p.du + (b * p.L) * p.Dm + d0;
    float *ddt_b = p.ddt + (b * p.L) * p.Dm + d0;
    const TIN *B_b = static_cast<const TIN *>(p.B) + (b * p.L) * p.N;
    const TIN *C_b = static_cast<const TIN *>(p.C) + (b * p.L) * p.N;
    float *ck_b = p.ck + (b * p.ntiles * p.Dm + d0) * p.N;
    float *pB_b = p.pB + ((cb * p.batch + b) * p.L) * p.N;
    float *pC_b = p.pC + ((cb * p.batch + b) * p.L) * p.N;
    const int Dm32 = (int)p.Dm, N32 = (int)p.N;
    const int cl = (int)(dcl - d0);                           // clamped channel within the block
    const uint32_t ck_off = (uint32_t)(((int)(dcn - d0) * N32 + (int)ncn) * 4);   // (d, n) in a tile's slab
    const uint32_t w_off = (uint32_t)(tl * Dm32 + c);          // element offset of outputs (t, d0 + c)
    const uint32_t p_off = (uint32_t)((tl * N32 + c) * 4);     // byte offset of dB/dC partials
    auto at = [](auto *base, uint32_t byte_off) __attribute__((always_inline)) {
        using T = std::remove_pointer_t<decltype(base)>;
        using C = std::conditional_t<std::is_const_v<T>, const char, char>;
        return reinterpret_cast<decltype(base)>(reinterpret_cast<C *>(base) + byte_off);
    };
    auto load_stage = [&](int kt, StageRaw &R, bool with_dy) __attribute__((always_inline)) {
        const int64_t t0 = (int64_t)kt * kT;
        const uint32_t e = (uint32_t)(min(tl, L - 1 - kt * kT) * Dm32 + cl);
        R.dt = *at(dt_b + t0 * p.Dm, e * 4u);
        R.u = In<TIN>::ld(at(u_b + t0 * p.Dm, e * (uint32_t)sizeof(TIN)), 0);
        if (with_dy) R.dy = *at(dy_b + t0 * p.Dm, e * 4u);
    };
    auto lane_e = [&](int kt) __attribute__((always_inline)) {
        return (uint32_t)(min(k, L - 1 - kt * kT) * N32 + (int)ncn);
    };
    auto load_lane = [&](int kt, LaneRaw &R, bool with_c) __attribute__((always_inline)) {
        const int64_t t0 = (int64_t)kt * kT;
        const uint32_t e = lane_e(kt);
        R.B = In<TIN>::ld(at(B_b + t0 * p.N, e * (uint32_t)sizeof(TIN)), 0);
        if (with_c) {
            R.C = In<TIN>::ld(at(C_b + t0 * p.N, e * (uint32_t)sizeof(TIN)), 0);
            R.hin = *at(ck_b + (int64_t)kt * ck_step_n(p), ck_off);
        }
    };
    // per-(t, d) values of the staged tile that the reduction phase needs
    float cur_dy = 0.0f, cur_sig = 0.0f, cur_u = 0.0f;
    auto stage = [&](int buf, int kt, const StageRaw &R, bool with_dy) __attribute__((always_inline)) {
        const bool tv = cok && kt * kT + tl < L;
        const float x = R.dt + bias;
        const float dl = tv ? softplus(x) : 0.0f;
        const float uv = tv ? R.u : 0.0f;
        sDl[buf][c][tl] = dl;
        sU[buf][c][tl] = uv;
        if (with_dy) {
            const float dyv = tv ? R.dy : 0.0f;
            sDy[buf][c][tl] = dyv;
            cur_dy = dyv;
            cur_u = uv;
            cur_sig = __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * kLog2e));   // sigmoid(x)
        }
    };
    // Abar and the input scale of one step: the forward's exact hold, so that
    // recomputed states equal the forward's bit for bit
    auto coef = [&](float dl) __attribute__((always_inline)) {
        Zoh zh = zoh_exact(dl, A, A2, iA);
        if constexpr (MODE == 1) zh.beta = dl;
        if constexpr (MODE == 2) zh.beta = 1.0f;
        return zh;
    };

    const float Bmask = n < p.N ? 1.0f : 0.0f;   // state-padding lanes carry zeros
    float h = (ok && p.h0) ? p.h0[(b * p.Dm + d) * p.N + n] : 0.0f;

    // ---- pass 1: forward, checkpointing the state entering each tile (or, with
    // the forward's saved states, only the last tile's loads and staging)
    StageRaw RS, RSn;
    LaneRaw RL, RLn;
    RS.dy = RSn.dy = 0.0f;
    RL.C = RL.hin = RLn.C = RLn.hin = 0.0f;
    if (p.saved) {
        const int kl = ntiles - 1;
        load_stage(kl, RS, true);
        load_lane(kl, RL, true);          // B, C and the saved state entering tile kl
        stage(kl & 1, kl, RS, true);
        h = ok ? RL.hin : 0.0f;
        __syncthreads();
    } else {
        load_stage(0, RS, ntiles == 1);
        load_lane(0, RL, false);
        stage(0, 0, RS, ntiles == 1);
        __syncthreads();
        for (int kt = 0; kt + 1 < ntiles; ++kt) {
            const int buf = kt & 1;
            if (ok) *at(ck_b + (int64_t)kt * ck_step_n(p), ck_off) = h;
            const bool last = kt + 2 == ntiles;            // the next tile is the last one
            load_stage(kt + 1, RSn, last);
            load_lane(kt + 1, RLn, false);
            if (last) RLn.C = In<TIN>::ld(at(C_b + (int64_t)(kt + 1) * kT * p.N, lane_e(kt + 1) * (uint32_t)sizeof(TIN)), 0);
            const float Bv = RL.B * Bmask;
            static_for<0, kT / 4>([&](auto qi) __attribute__((always_inline)) {
                constexpr int q = decltype(qi)::value;
                const float4 dq = *reinterpret_cast<const float4 *>(&sDl[buf][k][4 * q]);
                const float4 uq = *reinterpret_cast<const float4 *>(&sU[buf][k][4 * q]);
                const float dl4[4] = {dq.x, dq.y, dq.z, dq.w};
                const float uu4[4] = {uq.x, uq.y, uq.z, uq.w};
                static_for<0, 4>([&](auto ii) __attribute__((always_inline)) {
                    constexpr int i = decltype(ii)::value;
                    const Zoh zh = coef(dl4[i]);
                    const float bu = row_bcast<4 * q + i>(Bv) * uu4[i];
                    h = hold_step<MODE>(h, zh.ab, A, zh.beta, bu);
                });
            });
            stage(buf ^ 1, kt + 1, RSn, last);
            __syncthreads();
            RS = RSn;
            RL = RLn;
        }
        if (ntiles == 1) RL.C = In<TIN>::ld(at(C_b, lane_e(0) * (uint32_t)sizeof(TIN)), 0);
    }

    // ---- pass 2: backward over the tiles
    float g = (ok && p.dhf) ? p.dhf[(b * p.Dm + d) * p.N + n] : 0.0f;
    // dA_log / A = sum g (h_{t-1} delta Abar + B u dbeta/dA); kept as two sums:
    // dA1 = sum g Abar delta h_{t-1}, dA2 = A sum g B u dbeta/dA (times 1/A at the end)
    float dA1 = 0.0f, dA2 = 0.0f;
    float accD = 0.0f, accT = 0.0f;    // staging thread's sums of dy u and ddt over its steps
    float h_in = h;                     // state entering the last tile
    const int sw = n & 3;               // channel-chunk swizzle of this lane's dB/dC rows
    const int col = (((k >> 2) ^ sw) << 2) | (k & 3);
    for (int kt = ntiles - 1; kt >= 0; --kt) {
        const int buf = kt & 1;
        if (kt > 0) {
            load_stage(kt - 1, RSn, true);
            load_lane(kt - 1, RLn, true);
        }
        const float Bv = RL.B * Bmask, Cv = RL.C * Bmask;
        // recompute the tile's states hs[t] = h_t
        float hs[kT];
        {
            float hh = h_in;
            static_for<0, kT / 4>([&](auto qi) __attribute__((always_inline)) {
                constexpr int q = decltype(qi)::value;
                const float4 dq = *reinterpret_cast<const float4 *>(&sDl[buf][k][4 * q]);
                const float4 uq = *reinterpret_cast<const float4 *>(&sU[buf][k][4 * q]);
                const float dl4[4] = {dq.x, dq.y, dq.z, dq.w};
                const float uu4[4] = {uq.x, uq.y, uq.z, uq.w};
                static_for<0, 4>([&](auto ii) __attribute__((always_inline)) {
                    constexpr int i = decltype(ii)::value;
                    constexpr int t = 4 * q + i;
                    const Zoh zh = coef(dl4[i]);
                    const float bu = row_bcast<t>(Bv) * uu4[i];
                    hh = hold_step<MODE>(hh, zh.ab, A, zh.beta, bu);
                    hs[t] = hh;
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        // compiler-only fence: the adjoint re-reads delta, u from LDS and recomputes
        // Abar instead of keeping the recompute's values live (register pressure)
        asm volatile("" ::: "memory");
        // adjoint over the tile, last step first, in groups of 4 steps
        static_for<0, kT / 4>([&](auto ri) __attribute__((always_inline)) {
            constexpr int q = kT / 4 - 1 - decltype(ri)::value;
            const float4 dq = *reinterpret_cast<const float4 *>(&sDl[buf][k][4 * q]);
            const float4 uq = *reinterpret_cast<const float4 *>(&sU[buf][k][4 * q]);
            const float4 yq = *reinterpret_cast<const float4 *>(&sDy[buf][k][4 * q]);
            const float dl4[4] = {dq.x, dq.y, dq.z, dq.w};
            const float uu4[4] = {uq.x, uq.y, uq.z, uq.w};
            const float dy4[4] = {yq.x, yq.y, yq.z, yq.w};
            float pu[4], pd[4];
            static_for<0, 4>([&](auto ii) __attribute__((always_inline)) {
                constexpr int i = 3 - decltype(ii)::value;
                constexpr int t = 4 * q + i;
                const float dl = dl4[i], uu = uu4[i], dyv = dy4[i];
                const Zoh zh = coef(dl);
                const float ab = zh.ab;
                const float ht = hs[t];
                float hp;
                if constexpr (t > 0) hp = hs[t > 0 ? t - 1 : 0];
                else hp = h_in;
                const float Bt = row_bcast<t>(Bv);
                g = fmaf(row_bcast<t>(Cv), dyv, g);          // g_t = dL/dh_t
                const float beta = zh.beta;
                const float bu = Bt * uu;
                const float gb = g * beta;
                const float ga = g * ab;                     // g_t Abar_t: the cotangent passed to t - 1
                // the derivatives of Abar (A Abar, delta Abar) take the exponential itself: the
                // recurrence's 1 + A beta is accurate next to 1, but where a step's decay all but
                // erases the state it is off by ~1e-7 absolute against an Abar of e^{-25} or less
                const float ex = exp2_fast(dl * A2);
                const float gad = g * ex;
                // dB, dC terms of (t, n) from this channel
                sBC[0][t][n][col] = gb * uu;
                sBC[1][t][n][col] = dyv * ht;
                pu[i] = gb * Bt;
                if constexpr (MODE == 0) {
                    pd[i] = gad * fmaf(hp, A, bu);           // g Abar (A h_{t-1} + B u)
                    dA1 = fmaf(gad * dl, hp, dA1);
                    // A dbeta/dA = delta Abar - beta = delta z phi1'(z), z = delta A: the
                    // difference cancels to second order in z (relative error ~1e-7/z^2),
                    // so in the forward's series range it comes from the series of phi1'
                    const float z = dl * A;
                    const float w = dl * A2 > -kZohSeriesX ? dl * z * dphi1_series(z) : fmaf(dl, ex, -beta);
                    dA2 = fmaf(bu * g, w, dA2);
                } else if constexpr (MODE == 1) {
                    pd[i] = fmaf(gad, hp * A, g * bu);       // g (Abar A h_{t-1} + B u)
                    dA1 = fmaf(gad * dl, hp, dA1);
                } else {
                    pd[i] = gad * (hp * A);
                    dA1 = fmaf(gad * dl, hp, dA1);
                }
                g = ga;
            });
            const float su = rows_reduce4(pu[0], pu[1], pu[2], pu[3]);
            const float sd = rows_reduce4(pd[0], pd[1], pd[2], pd[3]);
            const int tr = 4 * q + ((rho & 1) ? 2 : 0) + (rho >> 1);
            sDD[wv][0][tr][k] = su;
            sDD[wv][1][tr][k] = sd;
            // keep the scheduler from hoisting later groups' work (register pressure)
            __builtin_amdgcn_sched_barrier(0);
        });
        __syncthreads();
        const bool tin = kt * kT + tl < L;
        // sums over states: thread (tl, c) -> du, ddt of (t, d0 + c)
        {
            const float su = (sDD[0][0][tl][c] + sDD[1][0][tl][c]) + (sDD[2][0][tl][c] + sDD[3][0][tl][c]);
            const float sd = (sDD[0][1][tl][c] + sDD[1][1][tl][c]) + (sDD[2][1][tl][c] + sDD[3][1][tl][c]);
            const float dtv = sd * cur_sig;
            if (cok && tin) {
                const int64_t o = (int64_t)kt * kT * p.Dm;
                *at(du_b + o, w_off * 4u) = fmaf(Dv, cur_dy, su);
                *at(ddt_b + o, w_off * 4u) = dtv;
                accD = fmaf(cur_dy, cur_u, accD);
                accT += dtv;
            }
        }
        // sums over the block's channels: thread (tl, s) -> dB, dC partials of (t, s)
        {
            const int s = c;
            const float4 *rb = reinterpret_cast<const float4 *>(&sBC[0][tl][s][0]);
            const float4 *rc = reinterpret_cast<const float4 *>(&sBC[1][tl][s][0]);
            float sb = 0.0f, sc = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 x = rb[j], y = rc[j];
                sb += (x.x + x.y) + (x.z + x.w);
                sc += (y.x + y.y) + (y.z + y.w);
            }
            if (tin && s < N32) {
                const int64_t o = (int64_t)kt * kT * p.N;
                *at(pB_b + o, p_off) = sb;
                *at(pC_b + o, p_off) = sc;
            }
        }
        if (kt > 0) stage(buf ^ 1, kt - 1, RSn, true);
        __syncthreads();
        if (kt > 0) {
            RL = RLn;
            h_in = RLn.hin;
        }
    }

    if (ok) {
        if (p.dh0) p.dh0[(b * p.Dm + d) * p.N + n] = g;
        p.pA[(b * p.Dm + d) * p.N + n] = fmaf(dA2, iA, dA1);
    }
    // per-channel sums of dy u and ddt over this batch row: the 16 staging
    // threads of channel c (tl = 0..15) hold partials
    sDD[0][0][tl][c] = accD;
    sDD[0][1][tl][c] = accT;
    __syncthreads();
    if (tl == 0 && cok) {
        float sD_ = 0.0f, sT_ = 0.0f;
#pragma unroll
        for (int i = 0; i < kT; ++i) { sD_ += sDD[0][0][i][c]; sT_ += sDD[0][1][i][c]; }
        p.pDv[b * p.Dm + dcs] = sD_;
        p.pTb[b * p.Dm + dcs] = sT_;
    }
}

template <typename TIN, int MODE>
__global__ void __launch_bounds__(kThreads, 3)
s6_bwd_kernel(S6BKp p) {
    __shared__ __attribute__((aligned(16))) Lds S;
    s6_bwd_body<TIN, MODE>(p, S);
}

// dB, dC = sum over channel blocks; dA_log = A * sum over batch; dD, ddt_bias = sum over batch
__global__ void __launch_bounds__(256)
s6_bwd_reduce_kernel(S6BKp p) {
    const int64_t nBC = p.batch * p.L * p.N, nA = p.Dm * p.N, nV = p.Dm;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < nBC) {
        float sb = 0.0f, sc = 0.0f;
        for (int64_t cb = 0; cb < p.ncblk; ++cb) { sb += p.pB[cb * nBC + i]; sc += p.pC[cb * nBC + i]; }
        p.dB[i] = sb;
        p.dC[i] = sc;
    } else if (i < nBC + nA) {
        const int64_t j = i - nBC;
        float s = 0.0f;
        for (int64_t bb = 0; bb < p.batch; ++bb) s += p.pA[bb * nA + j];
        p.dA_log[j] = s * -expf(p.A_log[j]);
    } else if (i < nBC + nA + nV) {
        const int64_t j = i - nBC - nA;
        float sD_ = 0.0f, sT_ = 0.0f;
        for (int64_t bb = 0; bb < p.batch; ++bb) { sD_ += p.pDv[bb * nV + j]; sT_ += p.pTb[bb * nV + j]; }
        if (p.dD) p.dD[j] = sD_;
        if (p.ddt_bias) p.ddt_bias[j] = sT_;
    }
}

struct WsLayout {
    size_t ck, pB, pC, pA, pDv, pTb, total;
};
size_t al256(size_t v) { return (v + 255) & ~size_t(255); }
WsLayout layout(int64_t batch, int64_t L, int64_t Dm, int64_t N) {
    const int64_t ntiles = (L + kT - 1) / kT, ncblk = (Dm + kCW - 1) / kCW;
    WsLayout w{};
    size_t o = 0;
    w.ck = o;  o += al256((size_t)(batch * ntiles * Dm * N) * 4);
    w.pB = o;  o += al256((size_t)(ncblk * batch * L * N) * 4);
    w.pC = o;  o += al256((size_t)(ncblk * batch * L * N) * 4);
    w.pA = o;  o += al256((size_t)(batch * Dm * N) * 4);
    w.pDv = o; o += al256((size_t)(batch * Dm) * 4);
    w.pTb = o; o += al256((size_t)(batch * Dm) * 4);
    w.total = o;
    return w;
}

template <typename TIN>
hipError_t launch_t(const S6BKp &p, int mode, hipStream_t s) {
    const dim3 grid((unsigned)(p.batch * p.ncblk)), block(kThreads);
    if (mode == 0) hipLaunchKernelGGL((s6_bwd_kernel<TIN, 0>), grid, block, 0, s, p);
    else if (mode == 1) hipLaunchKernelGGL((s6_bwd_kernel<TIN, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((s6_bwd_kernel<TIN, 2>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

size_t s6_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state) {
    return layout(batch, L, d_inner, d_state).total;
}

hipError_t launch_s6_bwd(const S6BwdArgs &a, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "s6_bwd_kernel";
    S6BKp p{};
    p.u = a.u; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C; p.D = a.D;
    p.h0 = a.h0; p.dy = a.dy; p.dhf = a.dh_final;
    p.du = a.du; p.ddt = a.ddt; p.dB = a.dB; p.dC = a.dC; p.dA_log = a.dA_log; p.dD = a.dD;
    p.ddt_bias = a.ddt_bias; p.dh0 = a.dh0;
    p.batch = a.batch; p.L = a.L; p.Dm = a.d_inner; p.N = a.d_state;
    p.ntiles = (a.L + kT - 1) / kT;
    p.ncblk = (a.d_inner + kCW - 1) / kCW;
    const WsLayout w = layout(a.batch, a.L, a.d_inner, a.d_state);
    char *ws = static_cast<char *>(a.workspace);
    p.ck = a.checkpoints ? const_cast<float *>(a.checkpoints) : reinterpret_cast<float *>(ws + w.ck);
    p.saved = a.checkpoints != nullptr;
    p.pB = reinterpret_cast<float *>(ws + w.pB);
    p.pC = reinterpret_cast<float *>(ws + w.pC);
    p.pA = reinterpret_cast<float *>(ws + w.pA);
    p.pDv = reinterpret_cast<float *>(ws + w.pDv);
    p.pTb = reinterpret_cast<float *>(ws + w.pTb);
    const int mode = (int)(a.flags & 0x3u);
    hipError_t e = a.bf16 ? launch_t<uint16_t>(p, mode, stream) : launch_t<float>(p, mode, stream);
    if (e != hipSuccess) return e;
    *kernel_name = "s6_bwd_reduce_kernel";
    const int64_t nred = p.batch * p.L * p.N + p.Dm * p.N + p.Dm;
    hipLaunchKernelGGL(s6_bwd_reduce_kernel, dim3((unsigned)((nred + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ssm
