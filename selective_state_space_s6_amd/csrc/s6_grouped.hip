// s6_grouped.hip -- the S6 forward scan with B, C per group of channels (per
// channel when the group count equals d_inner), gfx950.
//
// The recurrence is the selective scan's (builderforce-memory-engine
// selective_scan.js header comment, softplus, discretise_A/discretise_B,
// forward_scan + forward_reduce), with the input-dependent B and C read per
// channel: channel d takes row d * G / d_inner of B[b, t] and C[b, t].
//
// With one shared B row the main kernel hands B[t, n] to 16 channels by DPP
// broadcast.  Per-channel rows leave nothing to share, so here a 16-lane DPP
// row is ONE channel and lane k holds its states n = k + 16 j:
//  * every lane loads its own B, C values (a row reads a contiguous 64-byte
//    run of one step's row, a wave four channels' runs);
//  * dt and u of a 16-step tile are loaded one step per lane; lane k forms
//    delta = softplus(dt + dt_bias) of step k once, and both are handed to the
//    row with DPP row_newbcast as each step is scanned;
//  * the 16 per-step partial sums C.h of a tile are reduced over the row by a
//    4-stage butterfly that leaves step k's total in lane k, which adds D u
//    and writes y;
//  * the next tile's loads are in flight while a tile is scanned.
// The path moves 2 N values of B, C per (t, d) against 3 of u, dt, y: it is
// bound by HBM, not by the exp per state update.
#include "device_common.hpp"
#include "launchers.hpp"
#include <type_traits>
#include <utility>

namespace ssm {
namespace {

constexpr int kGT = 16;            // steps per tile == lanes per DPP row
constexpr int kGThreads = 256;     // 16 channels per work group
constexpr int kGChan = kGThreads / kGT;

// A lane's 32-bit byte offset, re-read where it is used: the empty asm keeps its
// zero extension next to the access, so that uniform base + offset is the global
// instructions' SGPR-base form rather than a 64-bit VALU add per access
__device__ __forceinline__ uint32_t g_lane_off(uint32_t o) {
    asm volatile("" : "+v"(o));
    return o;
}
template <typename T>
__device__ __forceinline__ T *g_at(T *base, uint32_t byte_off) {
    using Ch = std::conditional_t<std::is_const_v<T>, const char, char>;
    return reinterpret_cast<T *>(reinterpret_cast<Ch *>(base) + g_lane_off(byte_off));
}

template <int I, int N, typename F>
__device__ __forceinline__ void g_static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        g_static_for<I + 1, N>(f);
    }
}

struct S6Gp {
    const void *u; const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; float *y;
    const float *h0; float *h_final;
    int64_t batch, L, Dm, N, G;
    int64_t n_cblk;                // channel groups of 16 per batch row
    float *ck;                     // SAVE: (batch, ntiles, Dm, N), the state entering each tile
    int64_t ntiles;
};

// one tile's loads of one lane: B, C of its states at the tile's 16 steps, and
// dt, u of the step it stands for
template <int SPL>
struct GRaw {
    float B[kGT][SPL], C[kGT][SPL];
    float dt, u;
};

template <typename TIN, int SPL, int MODE, bool SAVE = false>
__global__ void __launch_bounds__(kGThreads)
s6_grouped_kernel(S6Gp p) {
    const int tid = threadIdx.x;
    const int k = tid & (kGT - 1);                      // lane in the row: state k + 16 j, step k
    const int64_t b = blockIdx.x / p.n_cblk;
    const int64_t d = (blockIdx.x % p.n_cblk) * kGChan + (tid >> 4);
    const bool dval = d < p.Dm;
    const int64_t dd = dval ? d : p.Dm - 1;             // clamped for loads
    const int64_t grp = dd * p.G / p.Dm;
    const int64_t rowBC = p.G * p.N;                    // B, C elements per step
    const TIN *Bb = static_cast<const TIN *>(p.B) + (b * p.L * p.G + grp) * p.N;
    const TIN *Cb = static_cast<const TIN *>(p.C) + (b * p.L * p.G + grp) * p.N;
    const TIN *Ub = static_cast<const TIN *>(p.u) + b * p.L * p.Dm + dd;
    const float *Db = p.dt + b * p.L * p.Dm + dd;

    int nidx[SPL];
    bool nval[SPL];
    float Av[SPL], A2[SPL], iA[SPL], h[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const int n = k + kGT * j;
        nval[j] = n < p.N;
        nidx[j] = nval[j] ? n : (int)p.N - 1;
        const bool ok = dval && nval[j];
        const float al = ok ? p.A_log[dd * p.N + n] : 0.0f;
        Av[j] = ok ? -fminf(expf(al), kMaxAbsA) : 0.0f;   // A = -exp(A_log)
        A2[j] = Av[j] * kLog2e;                            // A*log2(e)
        iA[j] = ok ? -expf(-al) : 0.0f;                    // 1/A
        h[j] = (ok && p.h0) ? p.h0[(b * p.Dm + d) * p.N + n] : 0.0f;
    }
    const float bias = (dval && p.dt_bias) ? p.dt_bias[dd] : 0.0f;
    const float Dd = (dval && p.D) ? p.D[dd] : 0.0f;

    // loads of the tile starting at t0; steps past L re-read step L-1 (their
    // delta and u are zeroed before use)
    auto load = [&](GRaw<SPL> &R, int64_t t0) __attribute__((always_inline)) {
        const int64_t last = p.L - 1 - t0;
#pragma unroll
        for (int s = 0; s < kGT; ++s) {
            const int64_t off = (s <= last ? s : last) * rowBC + t0 * rowBC;
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                R.B[s][j] = In<TIN>::ld(Bb, off + nidx[j]);
                R.C[s][j] = In<TIN>::ld(Cb, off + nidx[j]);
            }
        }
        const int64_t te = (k <= last ? k : last) + t0;
        R.dt = Db[te * p.Dm];
        R.u = In<TIN>::ld(Ub, te * p.Dm);
    };

    auto compute = [&](const GRaw<SPL> &R, int64_t t0) __attribute__((always_inline)) {
        if constexpr (SAVE) {
#pragma unroll
            for (int j = 0; j < SPL; ++j)
                if (dval && nval[j]) p.ck[((b * p.ntiles + t0 / kGT) * p.Dm + d) * p.N + k + kGT * j] = h[j];
        }
        const bool ok = dval && (t0 + k < p.L);
        const float dlk = ok ? softplus(R.dt + bias) : 0.0f;
        const float uk = ok ? R.u : 0.0f;
        float part[kGT];
        g_static_for<0, kGT>([&](auto ti) __attribute__((always_inline)) {
            constexpr int t = decltype(ti)::value;
            const float dl = row_bcast<t>(dlk);
            const float uu = row_bcast<t>(uk);
            float ys = 0.0f;
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const float bm = nval[j] ? R.B[t][j] : 0.0f;
                const float cm = nval[j] ? R.C[t][j] : 0.0f;
                const Zoh zh = zoh_exact(dl, Av[j], A2[j], iA[j]);   // Abar, (Abar - 1)/A
                const float beta = MODE == 0 ? zh.beta : MODE == 1 ? dl : 1.0f;
                h[j] = hold_step<MODE>(h[j], zh.ab, Av[j], beta, bm * uu);
                ys = fmaf(cm, h[j], ys);
            }
            part[t] = ys;
        });
        // butterfly over the row: after the stage of bit m a lane keeps the half
        // of the step indices whose bit m equals its own, summed with its partner
        g_static_for<0, 4>([&](auto si) __attribute__((always_inline)) {
            constexpr int M = 8 >> decltype(si)::value;
            const bool up = (k & M) != 0;
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const float send = up ? part[i] : part[i + M];
                const float keep = up ? part[i + M] : part[i];
                part[i] = keep + __shfl_xor(send, M, kGT);
            }
        });
        if (ok) p.y[(b * p.L + t0 + k) * p.Dm + d] = fmaf(Dd, uk, part[0]);
    };

    const int64_t ntiles = (p.L + kGT - 1) / kGT;
    GRaw<SPL> RA, RB;
    load(RA, 0);
    if (ntiles > 1) load(RB, kGT);
    for (int64_t kt = 0; kt < ntiles; kt += 2) {
        compute(RA, kt * kGT);
        if (kt + 2 < ntiles) load(RA, (kt + 2) * kGT);
        if (kt + 1 < ntiles) {
            compute(RB, (kt + 1) * kGT);
            if (kt + 3 < ntiles) load(RB, (kt + 3) * kGT);
        }
    }
    if (p.h_final && dval) {
#pragma unroll
        for (int j = 0; j < SPL; ++j)
            if (nval[j]) p.h_final[(b * p.Dm + d) * p.N + k + kGT * j] = h[j];
    }
}

template <typename TIN, int SPL, bool SAVE = false>
void launch_mode(const S6Gp &p, int mode, hipStream_t s) {
    const dim3 grid((unsigned)(p.batch * p.n_cblk)), block(kGThreads);
    if (mode == 0) hipLaunchKernelGGL((s6_grouped_kernel<TIN, SPL, 0, SAVE>), grid, block, 0, s, p);
    else if (mode == 1) hipLaunchKernelGGL((s6_grouped_kernel<TIN, SPL, 1, SAVE>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((s6_grouped_kernel<TIN, SPL, 2, SAVE>), grid, block, 0, s, p);
}

template <typename TIN>
void launch_spl(const S6Gp &p, int mode, hipStream_t s) {
    if (p.N <= kGT) launch_mode<TIN, 1>(p, mode, s);
    else launch_mode<TIN, 2>(p, mode, s);
}

// ---------------------------------------------------------------- backward
// The backward of the scan above: the reverse-time chain rule of the
// selective scan page's backward_scan (builderforce-memory-engine
// selective_scan.js), completed with beta's dependence on A, with B and C read
// per channel and dB, dC kept per channel (summed over a group's channels by
// s6_grouped_bwd_reduce when groups hold several).  The lane map is the
// forward's (a DPP row is a channel, lane k holds state k; N <= 16):
//   pass 1  forward over 16-step tiles, saving the state entering each tile;
//   pass 2  backward over the tiles: the tile's 16 states recomputed from its
//           saved state, then the adjoint, last step first.  Per step a lane
//           forms its state's dB = g beta u and dC = dy h (stored directly),
//           its shares of du and ddt (summed over the row by the butterfly,
//           step k's totals in lane k) and its dA term.
// dA_log, dD, ddt_bias go through per-batch-row partials, added in a fixed
// order by s6_grouped_bwd_reduce.

struct S6GBp {
    const void *u; const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; const float *h0;
    const float *dy; const float *dhf;
    float *du, *ddt, *dh0;
    float *dBw, *dCw;            // (batch, L, Dm, N): per-channel dB, dC (the outputs when G = Dm)
    float *dB, *dC;              // (batch, L, G, N)
    float *dA_log, *dD, *ddt_bias;
    float *ck;                   // (batch, ntiles, Dm, N)
    float *pA, *pD, *pT;         // (batch, Dm, N), (batch, Dm), (batch, Dm)
    int64_t batch, L, Dm, N, G, ntiles, n_cblk;
    bool saved;                  // ck holds the forward's saved states: no pass 1
};

// phi1'(z) to z^3 (|z| < 1/8: truncation < 4e-6 relative)
__device__ __forceinline__ float g_dphi1_small(float z) {
    float q = fmaf(z, 1.0f / 30.0f, 1.0f / 8.0f);
    q = fmaf(z, q, 1.0f / 3.0f);
    return fmaf(z, q, 0.5f);
}

// 16 per-step values of each lane of a row -> lane k holds the row's total of step k
__device__ __forceinline__ float g_row_transpose_sum(float (&part)[kGT], int k) {
    g_static_for<0, 4>([&](auto si) __attribute__((always_inline)) {
        constexpr int M = 8 >> decltype(si)::value;
        const bool up = (k & M) != 0;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const float send = up ? part[i] : part[i + M];
            const float keep = up ? part[i + M] : part[i];
            part[i] = keep + __shfl_xor(send, M, kGT);
        }
    });
    return part[0];
}

struct GBRaw {
    float B[kGT], C[kGT];
    float dt, u, dy;
};

template <typename TIN, int MODE>
__device__ __forceinline__ void s6_grouped_bwd_body(const S6GBp &p) {
    const int tid = threadIdx.x;
    const int k = tid & (kGT - 1);                      // state k, step k of a tile
    const int64_t b = blockIdx.x / p.n_cblk;
    const int64_t d0 = (blockIdx.x % p.n_cblk) * kGChan;
    const int c = tid >> 4;                             // channel within the group
    const int64_t d = d0 + c;
    const bool dval = d < p.Dm;
    const int64_t dd = dval ? d : p.Dm - 1;
    const bool nval = k < p.N;
    const int64_t nn = nval ? k : p.N - 1;
    const bool ok = dval && nval;
    const int64_t grp = dd * p.G / p.Dm;
    const int64_t rowBC = p.G * p.N;
    const int64_t L = p.L, ntiles = p.ntiles;
    // Addresses: a block-uniform base (scalar registers) plus a 32-bit per-lane byte
    // offset, so the unrolled steps share one offset register each (the caller
    // bounds d_inner * d_state, so every offset below stays far below 4 GiB)
    const uint32_t o_bc = (uint32_t)((grp * p.N + nn) * (int64_t)sizeof(TIN));   // within a step's B, C row
    const uint32_t o_ck = (uint32_t)((dd * p.N + nn) * 4);                         // within a tile's saved states
    const uint32_t o_dbc = (uint32_t)(((int64_t)c * p.N + k) * 4);                 // within a step's dB, dC rows of the group's channels
    const uint32_t o_ch = (uint32_t)(dd * 4);                                      // within a step's row of d_inner (fp32)
    const uint32_t o_chi = (uint32_t)(dd * (int64_t)sizeof(TIN));                  // the same for u
    auto at = [](auto *base, uint32_t byte_off) __attribute__((always_inline)) { return g_at(base, byte_off); };
    const TIN *Bb = static_cast<const TIN *>(p.B) + b * L * rowBC;
    const TIN *Cb = static_cast<const TIN *>(p.C) + b * L * rowBC;
    const TIN *Ub = static_cast<const TIN *>(p.u) + b * L * p.Dm;
    const float *Db = p.dt + b * L * p.Dm;
    const float *DYb = p.dy + b * L * p.Dm;

    const float al = ok ? p.A_log[dd * p.N + nn] : 0.0f;
    const float A = ok ? -fminf(expf(al), kMaxAbsA) : 0.0f;
    const float A2 = A * kLog2e;
    const float iA = ok ? -expf(-al) : 0.0f;
    const float bias = (dval && p.dt_bias) ? p.dt_bias[dd] : 0.0f;
    const float Dd = (dval && p.D) ? p.D[dd] : 0.0f;

    auto load = [&](GBRaw &R, int64_t kt, bool full) __attribute__((always_inline)) {
        const int64_t t0 = kt * kGT, last = L - 1 - t0;
#pragma unroll
        for (int s = 0; s < kGT; ++s) {
            const int64_t off = ((s <= last ? s : last) + t0) * rowBC;   // uniform
            R.B[s] = In<TIN>::ld(at(Bb + off, o_bc), 0);
            R.C[s] = full ? In<TIN>::ld(at(Cb + off, o_bc), 0) : 0.0f;
        }
        // step k of the tile: a uniform row base plus this lane's row and channel
        const uint32_t ok_row = (uint32_t)(k <= last ? k : last);
        const uint32_t step_f = ok_row * (uint32_t)p.Dm * 4u, step_i = ok_row * (uint32_t)p.Dm * (uint32_t)sizeof(TIN);
        R.dt = *at(Db + t0 * p.Dm, step_f + o_ch);
        R.u = In<TIN>::ld(at(Ub + t0 * p.Dm, step_i + o_chi), 0);
        R.dy = full ? *at(DYb + t0 * p.Dm, step_f + o_ch) : 0.0f;
    };
    // Abar and the input scale of one step: the forward's exact hold, so that
    // recomputed states equal the forward's bit for bit
    auto coef = [&](float dl) __attribute__((always_inline)) {
        Zoh zh = zoh_exact(dl, A, A2, iA);
        if constexpr (MODE == 1) zh.beta = dl;
        if constexpr (MODE == 2) zh.beta = 1.0f;
        return zh;
    };

    // ---- pass 1: the state entering each tile (unless the forward saved them)
    float *ck_b = p.ck + b * ntiles * p.Dm * p.N;         // + tile * Dm * N, + o_ck
    if (!p.saved) {
        float h = (ok && p.h0) ? p.h0[(b * p.Dm + d) * p.N + k] : 0.0f;
        GBRaw RA, RB;
        load(RA, 0, false);
        if (ntiles > 1) load(RB, 1, false);
        auto step1 = [&](GBRaw &R, int64_t kt) __attribute__((always_inline)) {
            if (ok) *at(ck_b + kt * p.Dm * p.N, o_ck) = h;
            const bool sv = dval && kt * kGT + k < L;
            const float dlk = sv ? softplus(R.dt + bias) : 0.0f;
            const float uk = sv ? R.u : 0.0f;
            g_static_for<0, kGT>([&](auto ti) __attribute__((always_inline)) {
                constexpr int t = decltype(ti)::value;
                const float dl = row_bcast<t>(dlk), uu = row_bcast<t>(uk);
                const Zoh zh = coef(dl);
                const float bm = nval ? R.B[t] : 0.0f;
                h = hold_step<MODE>(h, zh.ab, A, zh.beta, bm * uu);
            });
        };
        for (int64_t kt = 0; kt < ntiles; kt += 2) {
            step1(RA, kt);
            if (kt + 2 < ntiles) load(RA, kt + 2, false);
            if (kt + 1 < ntiles) {
                step1(RB, kt + 1);
                if (kt + 3 < ntiles) load(RB, kt + 3, false);
            }
        }
    }
    // a lane reads back only the states of its own (channel, state): written by
    // itself in pass 1, or by the forward's lane of the same pair

    // ---- pass 2: backward over the tiles
    float g = (ok && p.dhf) ? p.dhf[(b * p.Dm + d) * p.N + k] : 0.0f;
    float accA = 0.0f, accD = 0.0f, accT = 0.0f;
    auto step2 = [&](GBRaw &R, int64_t kt) __attribute__((always_inline)) {
        const int64_t t0 = kt * kGT;
        // lanes without a state start from 0 (their clamped slot is another lane's)
        const float h_in = ok ? *at(ck_b + kt * p.Dm * p.N, o_ck) : 0.0f;
        const bool sv = dval && t0 + k < L;
        const float x = R.dt + bias;
        const float dlk = sv ? softplus(x) : 0.0f;
        const float uk = sv ? R.u : 0.0f;
        const float dyk = sv ? R.dy : 0.0f;
        const float sgk = __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * kLog2e));   // sigmoid(x)
        float hs[kGT];
        {
            float hh = h_in;
            g_static_for<0, kGT>([&](auto ti) __attribute__((always_inline)) {
                constexpr int t = decltype(ti)::value;
                const float dl = row_bcast<t>(dlk), uu = row_bcast<t>(uk);
                const Zoh zh = coef(dl);
                const float bm = nval ? R.B[t] : 0.0f;
                hh = hold_step<MODE>(hh, zh.ab, A, zh.beta, bm * uu);
                hs[t] = hh;
            });
        }
        // compiler-only fence: the adjoint recomputes Abar and beta rather than keeping
        // the recompute's 32 values live (register pressure)
        asm volatile("" ::: "memory");
        float pu[kGT], pd[kGT];
        g_static_for<0, kGT>([&](auto ri) __attribute__((always_inline)) {
            constexpr int t = kGT - 1 - decltype(ri)::value;
            const float dl = row_bcast<t>(dlk), uu = row_bcast<t>(uk), dyv = row_bcast<t>(dyk);
            const Zoh zh = coef(dl);
            const float ab = zh.ab, beta = zh.beta;
            // the derivatives of Abar and beta take the exponential itself: 1 + A beta, which
            // the recurrence keeps, is off by ~1e-7 absolute where Abar is e^{-25} or less
            const float ex = exp2_fast(dl * A2);
            float bD, bA;
            if constexpr (MODE == 0) {
                bD = ex;
                // dbeta/dA = (delta Abar - beta)/A cancels to second order in z, so in
                // the forward's series range it comes from the series of phi1'
                const float z = dl * A;
                bA = dl * A2 > -kZohSeriesX ? dl * dl * g_dphi1_small(z) : (dl * ex - beta) * iA;
            } else if constexpr (MODE == 1) {
                bD = 1.0f; bA = 0.0f;
            } else {
                bD = 0.0f; bA = 0.0f;
            }
            const float bm = nval ? R.B[t] : 0.0f, cm = nval ? R.C[t] : 0.0f;
            g = fmaf(cm, dyv, g);
            const float hp = t > 0 ? hs[t > 0 ? t - 1 : 0] : h_in;
            const float bu = bm * uu;
            const float gb = g * beta;
            if (ok && t0 + t < L) {
                const int64_t row = ((b * L + t0 + t) * p.Dm + d0) * p.N;   // uniform
                *at(p.dBw + row, o_dbc) = gb * uu;
                *at(p.dCw + row, o_dbc) = dyv * hs[t];
            }
            pu[t] = gb * bm;
            pd[t] = g * fmaf(hp * A, ex, bu * bD);
            accA = fmaf(g, fmaf(hp * dl, ex, bu * bA), accA);
            g *= ab;
        });
        const float su = g_row_transpose_sum(pu, k);
        const float sd = g_row_transpose_sum(pd, k);
        if (sv) {
            const float ddt = sd * sgk;
            const uint32_t ob = (uint32_t)k * (uint32_t)p.Dm * 4u + o_ch;        // step k, channel d
            *at(p.du + (b * L + t0) * p.Dm, ob) = fmaf(Dd, dyk, su);
            *at(p.ddt + (b * L + t0) * p.Dm, ob) = ddt;
            accD = fmaf(dyk, uk, accD);
            accT += ddt;
        }
    };
    {
        GBRaw RA, RB;
        const int64_t kl = ntiles - 1;
        load(RA, kl, true);
        if (kl >= 1) load(RB, kl - 1, true);
        for (int64_t kt = kl; kt >= 0; kt -= 2) {
            step2(RA, kt);
            if (kt - 2 >= 0) load(RA, kt - 2, true);
            if (kt - 1 >= 0) {
                step2(RB, kt - 1);
                if (kt - 3 >= 0) load(RB, kt - 3, true);
            }
        }
    }
    if (ok && p.dh0) p.dh0[(b * p.Dm + d) * p.N + k] = g;
    if (ok) p.pA[(b * p.Dm + d) * p.N + k] = accA;
    // dD, ddt_bias of the channel: its lanes hold disjoint steps; a fixed-order row sum
    g_static_for<0, 4>([&](auto si) __attribute__((always_inline)) {
        constexpr int M = 8 >> decltype(si)::value;
        accD += __shfl_xor(accD, M, kGT);
        accT += __shfl_xor(accT, M, kGT);
    });
    if (dval && k == 0) {
        p.pD[b * p.Dm + d] = accD;
        p.pT[b * p.Dm + d] = accT;
    }
}

template <typename TIN, int MODE>
__global__ void __launch_bounds__(kGThreads)
s6_grouped_bwd_kernel(S6GBp p) {
    s6_grouped_bwd_body<TIN, MODE>(p);
}

// dB, dC over each group's channels (when a group holds several); dA_log = A * sum over
// the batch; dD, ddt_bias = sums over the batch; all in a fixed order
__global__ void __launch_bounds__(256) s6_grouped_bwd_reduce(S6GBp p) {
    const int64_t nBC = p.Dm == p.G ? 0 : p.batch * p.L * p.G * p.N, nA = p.Dm * p.N, nV = p.Dm;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < nBC) {
        const int64_t n = i % p.N, bt = i / p.N / p.G, gq = (i / p.N) % p.G;
        const int64_t cpg = p.Dm / p.G;
        float sb = 0.0f, sc = 0.0f;
        for (int64_t j = 0; j < cpg; ++j) {
            const int64_t o = (bt * p.Dm + gq * cpg + j) * p.N + n;
            sb += p.dBw[o];
            sc += p.dCw[o];
        }
        p.dB[i] = sb;
        p.dC[i] = sc;
    } else if (i < nBC + nA) {
        const int64_t j = i - nBC;
        float s_ = 0.0f;
        for (int64_t bb = 0; bb < p.batch; ++bb) s_ += p.pA[bb * nA + j];
        p.dA_log[j] = s_ * -expf(p.A_log[j]);
    } else if (i < nBC + nA + nV) {
        const int64_t j = i - nBC - nA;
        float sD_ = 0.0f, sT_ = 0.0f;
        for (int64_t bb = 0; bb < p.batch; ++bb) { sD_ += p.pD[bb * nV + j]; sT_ += p.pT[bb * nV + j]; }
        if (p.dD) p.dD[j] = sD_;
        if (p.ddt_bias) p.ddt_bias[j] = sT_;
    }
}

struct GBLayout { size_t ck, pA, pD, pT, dBw, dCw, total; };
size_t g_al256(size_t v) { return (v + 255) & ~size_t(255); }
GBLayout gb_layout(int64_t batch, int64_t L, int64_t Dm, int64_t N, int64_t G) {
    const int64_t ntiles = (L + kGT - 1) / kGT;
    GBLayout w{};
    size_t o = 0;
    w.ck = o;  o += g_al256((size_t)(batch * ntiles * Dm * N) * 4);
    w.pA = o;  o += g_al256((size_t)(batch * Dm * N) * 4);
    w.pD = o;  o += g_al256((size_t)(batch * Dm) * 4);
    w.pT = o;  o += g_al256((size_t)(batch * Dm) * 4);
    const size_t sh = G == Dm ? 0 : (size_t)(batch * L * Dm * N) * 4;   // per-channel shares
    w.dBw = o; o += g_al256(sh);
    w.dCw = o; o += g_al256(sh);
    w.total = o;
    return w;
}

}  // namespace

size_t s6_grouped_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups) {
    if (ngroups == 1) return s6_bwd_workspace_bytes(batch, L, d_inner, d_state);
    return gb_layout(batch, L, d_inner, d_state, ngroups).total;
}

hipError_t launch_s6_grouped_bwd(const S6BwdArgs &a, int64_t ngroups, hipStream_t stream, const char **kernel_name) {
    if (ngroups == 1) return launch_s6_bwd(a, stream, kernel_name);
    *kernel_name = "s6_grouped_bwd_kernel";
    S6GBp p{};
    p.u = a.u; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C; p.D = a.D;
    p.h0 = a.h0; p.dy = a.dy; p.dhf = a.dh_final;
    p.du = a.du; p.ddt = a.ddt; p.dh0 = a.dh0; p.dB = a.dB; p.dC = a.dC;
    p.dA_log = a.dA_log; p.dD = a.dD; p.ddt_bias = a.ddt_bias;
    p.batch = a.batch; p.L = a.L; p.Dm = a.d_inner; p.N = a.d_state; p.G = ngroups;
    p.ntiles = (a.L + kGT - 1) / kGT;
    p.n_cblk = (a.d_inner + kGChan - 1) / kGChan;
    const GBLayout w = gb_layout(a.batch, a.L, a.d_inner, a.d_state, ngroups);
    char *ws = static_cast<char *>(a.workspace);
    p.saved = a.checkpoints != nullptr;
    p.ck = p.saved ? const_cast<float *>(a.checkpoints) : reinterpret_cast<float *>(ws + w.ck);
    p.pA = reinterpret_cast<float *>(ws + w.pA);
    p.pD = reinterpret_cast<float *>(ws + w.pD);
    p.pT = reinterpret_cast<float *>(ws + w.pT);
    p.dBw = ngroups == a.d_inner ? a.dB : reinterpret_cast<float *>(ws + w.dBw);
    p.dCw = ngroups == a.d_inner ? a.dC : reinterpret_cast<float *>(ws + w.dCw);
    const int mode = (int)(a.flags & 0x3u);
    const dim3 grid((unsigned)(p.batch * p.n_cblk)), block(kGThreads);
    if (a.bf16) {
        if (mode == 0) hipLaunchKernelGGL((s6_grouped_bwd_kernel<uint16_t, 0>), grid, block, 0, stream, p);
        else if (mode == 1) hipLaunchKernelGGL((s6_grouped_bwd_kernel<uint16_t, 1>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((s6_grouped_bwd_kernel<uint16_t, 2>), grid, block, 0, stream, p);
    } else {
        if (mode == 0) hipLaunchKernelGGL((s6_grouped_bwd_kernel<float, 0>), grid, block, 0, stream, p);
        else if (mode == 1) hipLaunchKernelGGL((s6_grouped_bwd_kernel<float, 1>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((s6_grouped_bwd_kernel<float, 2>), grid, block, 0, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    *kernel_name = "s6_grouped_bwd_reduce";
    const int64_t nred = (ngroups == a.d_inner ? 0 : p.batch * p.L * p.G * p.N) + p.Dm * p.N + p.Dm;
    hipLaunchKernelGGL(s6_grouped_bwd_reduce, dim3((unsigned)((nred + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_s6_grouped(const S6Args &a, int64_t ngroups, hipStream_t stream, const char **kernel_name) {
    if (ngroups == 1) return launch_s6(a, stream, kernel_name);
    *kernel_name = "s6_grouped_kernel";
    S6Gp p{};
    p.u = a.u; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C;
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.Dm = a.d_inner; p.N = a.d_state; p.G = ngroups;
    p.n_cblk = (a.d_inner + kGChan - 1) / kGChan;
    const int mode = (int)(a.flags & 0x3u);
    if (a.bf16) launch_spl<uint16_t>(p, mode, stream);
    else launch_spl<float>(p, mode, stream);
    return hipGetLastError();
}

hipError_t launch_s6_grouped_save(const S6Args &a, int64_t ngroups, float *checkpoints, hipStream_t stream,
                                  const char **kernel_name) {
    if (ngroups == 1) return launch_s6_save(a, checkpoints, stream, kernel_name);
    *kernel_name = "s6_grouped_kernel";
    S6Gp p{};
    p.u = a.u; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C;
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.Dm = a.d_inner; p.N = a.d_state; p.G = ngroups;
    p.n_cblk = (a.d_inner + kGChan - 1) / kGChan;
    p.ck = checkpoints;
    p.ntiles = (a.L + kGT - 1) / kGT;
    const int mode = (int)(a.flags & 0x3u);
    // d_state <= 16 (the backward's limit): one state per lane
    if (a.bf16) launch_mode<uint16_t, 1, true>(p, mode, stream);
    else launch_mode<float, 1, true>(p, mode, stream);
    return hipGetLastError();
}

}  // namespace ssm
