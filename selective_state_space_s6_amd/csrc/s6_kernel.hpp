// s6_kernel.hpp -- the Mamba-1 (S6) forward selective scan kernel for gfx950,
// instantiated plain in s6_scan.hip and in its fused layer form in s6_fused.hip.
//
// Computes, per batch b and channel d, the diagonal recurrence of
// builderforce-memory-engine selective_scan.js (header comment, softplus,
// discretise_A/discretise_B, forward_scan + forward_reduce) and mamba-rs 0.4.0
// forward.rs step F4d, in ONE kernel: softplus of dt, exact zero-order-hold
// discretisation, the recurrence over time, the reduction over the state index
// and the D skip term.  Nothing but y (and h_final) is written to memory.
//
// Work decomposition (the path is bound by VALU issue, not by HBM: every
// (t, d, n) needs one exp, the exact hold's series and select, and ~6 more fp32
// operations, about 17 issue slots):
//  * a 256-thread block owns CW = 256/G channels of one batch row and walks the
//    whole sequence in tiles of 16 time steps;
//  * the N states of a channel are spread over G lanes (SPL = N/G states per
//    lane), so G*CW = 256 lanes each hold a few states in registers;
//  * a 16-lane DPP row is 16 channels that share one state group; B[t, n] and
//    C[t, n] of the 16 steps of a tile are held one step per lane and handed
//    to the whole row with DPP row_newbcast, folded into the multiply;
//  * delta = softplus(dt + dt_bias) and u are staged once per (t, d) through LDS
//    (b128 reads), the per-lane partial sums C.h go back through LDS and one
//    thread per (t, d) adds the G partials, adds D*u and writes y;
//  * global loads of the tile after next are in flight while a tile is scanned.
//
// Segmented form (PASS 1 and 3; the plain sequential walk is PASS 0): for long
// sequences over few channels, time is cut into segments of seg_len steps.
// PASS 1 runs each segment but the last from a zero state and writes its local
// final state and its sum of delta (the segment's decay is exp(A * sum)); a
// carry kernel combines the (decay, state) pairs with the associative rule
// (earlier, then later: (P2 P1, P2 h1 + h2)) into every segment's entering
// state; PASS 3 scans each segment from that state and writes y (and, in the
// last segment, h_final).  selective_scan.js forward_scan carries a tile's
// state the same way (its printed combine has the order reversed).
//
// Fused layer form (FUSE): the kernel reads x instead of u and forms
// u_t = SiLU(sum_k conv_w[d,k] x_{t-k} + conv_b[d]) as it stages a tile (the
// three earlier steps are cache hits, the carried conv state stands in before
// step 0), and multiplies each output by SiLU(z) as it writes y.
#pragma once
#include "device_common.hpp"
#include "launchers.hpp"
#include <algorithm>
#include <type_traits>
#include <utility>

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr int kT = 16;        // time steps per tile == lanes per DPP row
constexpr int kTS = kT + 4;   // padded LDS row: conflict-free b128 reads by 16 lanes

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

struct S6Kp {
    const void *u; const float *dt; const float *dt_bias; const float *A_log;
    const void *B; const void *C; const float *D; float *y;
    const float *h0; float *h_final;
    int64_t batch, L, Dm, N;
    int64_t n_cblk;   // channel blocks per batch row
    // fused layer form (FUSE): u is x, u_t = SiLU(sum_k conv_w[d,k] x_{t-k} + conv_b[d])
    // with x_{t<0} from conv_state (batch, Dm, K-1); y is multiplied by SiLU(z)
    const float *conv_w, *conv_b, *conv_state;
    const void *z;
    float *u_out;
    int K;
    // SAVE form: the state entering every 16-step tile, (batch, ntiles, Dm, N) fp32
    // (the saved states the S6 backward reads in place of recomputing them)
    float *ck;
    // segmented form: nseg segments of seg_len steps (the last may be shorter);
    // PASS 1 writes h_loc (batch, nseg-1, Dm, N) and dsum (batch, nseg-1, Dm),
    // PASS 3 reads h_in (batch, nseg, Dm, N)
    int64_t seg_len, nseg;
    float *h_loc;
    double *dsum;
    const float *h_in;
};

constexpr int kMaxConv = 4;   // longest causal convolution of the fused form

template <int EPT>
struct FuseRaw {      // the fused form's extra inputs of one tile
    float xh[EPT][kMaxConv - 1];   // x at t-1, t-2, t-3
    float z[EPT];
};
struct NoFuse {};

template <typename TIN, int G, int SPL, bool FUSE>
struct Raw {          // one tile of raw inputs held in registers
    float dt[16 / G];
    float u[16 / G];  // u, or x in the fused form
    float B[SPL];
    float C[SPL];
    std::conditional_t<FUSE, FuseRaw<16 / G>, NoFuse> f;
};

// Per-thread base pointers of the tensors this thread loads or stores, at
// time step 0 of the block's channels; a tile adds a uniform 64-bit offset.
template <typename TIN, int G, int SPL>
struct Ptrs {
    const float *dt[16 / G];
    const TIN *u[16 / G];
    const TIN *z[16 / G];   // fused form: z (or u when there is no gate)
    float *y[16 / G];
    const TIN *B;     // row t = k (this lane's step in a tile), column 0
    const TIN *C;
    int nidx[SPL];    // this lane's state columns, clamped into [0, N)
};

// Loads of one tile.  They are unconditional so the compiler can keep them in
// flight across the scan of the previous tile.  A tile that may cross L
// (CHECK) clamps its time index into the tensors; values of steps past L,
// channels past d_inner and states past N are masked where they are consumed
// (channel and state indices are clamped once, in the base pointers).
template <bool CHECK, bool WITH_C, typename TIN, int G, int SPL, bool FUSE>
__device__ __forceinline__ void load_raw(Raw<TIN, G, SPL, FUSE> &r, const Ptrs<TIN, G, SPL> &q,
                                         const S6Kp &p, int64_t Lk, int64_t t0, int tid, int k) {
    constexpr int CW = kThreads / G;
    constexpr int EPT = 16 / G;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int tl = (tid + kThreads * i) / CW;
        int64_t off = t0 * p.Dm;
        if constexpr (CHECK) off = (min(t0 + tl, Lk - 1) - tl) * p.Dm;
        r.dt[i] = q.dt[i][off];
        r.u[i] = In<TIN>::ld(q.u[i], off);
        if constexpr (FUSE) {
            // the three steps before: cache hits, as neighbouring lanes load them as
            // their own step; times before 0 are clamped here and replaced by the
            // carried state when staged
#pragma unroll
            for (int kk = 1; kk < kMaxConv; ++kk) {
                int64_t offk = t0 * p.Dm - kk * p.Dm;
                if constexpr (CHECK) offk = (max(min(t0 + tl, Lk - 1) - kk, (int64_t)0) - tl) * p.Dm;
                r.f.xh[i][kk - 1] = In<TIN>::ld(q.u[i], offk);
            }
            r.f.z[i] = In<TIN>::ld(q.z[i], off);
        }
    }
    int64_t off = t0 * p.N;
    if constexpr (CHECK) off = (min(t0 + k, Lk - 1) - k) * p.N;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        r.B[j] = In<TIN>::ld(q.B, off + q.nidx[j]);
        r.C[j] = WITH_C ? In<TIN>::ld(q.C, off + q.nidx[j]) : 0.0f;
    }
}

template <typename TIN, int G, int SPL, int MODE, bool FUSE, bool SAVE = false, int PASS = 0>
__global__ void __launch_bounds__(kThreads)
s6_scan_kernel(S6Kp p) {
    static_assert(PASS == 0 || PASS == 1 || PASS == 3, "PASS: 0 whole sequence, 1 segment states, 3 segment scan");
    static_assert(PASS == 0 || (!FUSE && !SAVE), "the segmented form is the plain scan");
    constexpr bool YOUT = PASS != 1;     // this pass forms y
    constexpr int CW = kThreads / G;     // channels per block
    constexpr int EPT = 16 / G;          // (t, d) elements per thread per tile
    __shared__ __attribute__((aligned(16))) float sD[2][CW][kTS];
    __shared__ __attribute__((aligned(16))) float sU[2][CW][kTS];
    // per-state-group partial sums C.h of a tile, [g][t * CW + channel]: a wave's
    // writes cover 4 state groups at once, so the group stride is padded by 16
    // floats off a multiple of the 64 banks (no 4-way write conflict); the
    // reduction reads 64 consecutive floats of one group
    constexpr int kYS = kT * CW + 16;
    __shared__ __attribute__((aligned(16))) float sY[2][G][kYS];

    const int tid = threadIdx.x;
    const int row = tid >> 4, k = tid & 15;
    const int g = row % G;
    const int cl = (row / G) * 16 + k;                 // this lane's channel in the block
    const int64_t work = xcd_swizzle(blockIdx.x, gridDim.x);
    // segmented form: work = (segment, batch row, channel block), channel block fastest
    const int64_t seg = PASS == 0 ? 0 : work / (p.batch * p.n_cblk);
    const int64_t rest = PASS == 0 ? work : work % (p.batch * p.n_cblk);
    const int64_t b = rest / p.n_cblk;
    const int64_t d0 = (rest % p.n_cblk) * CW;
    const int64_t d = d0 + cl;
    const bool dok = d < p.Dm;
    const int64_t T0 = seg * p.seg_len;                               // first step of this block
    const int64_t Lk = PASS == 0 ? p.L : min(p.seg_len, p.L - T0);    // steps of this block

    // per-lane constants of the states this lane owns
    float Av[SPL], A2[SPL], iA[SPL], h[SPL];
    bool nval[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const int64_t n = (int64_t)g * SPL + j;
        nval[j] = n < p.N;
        const bool ok = dok && n < p.N;
        const float al = ok ? p.A_log[d * p.N + n] : 0.0f;
        Av[j] = ok ? -fminf(expf(al), kMaxAbsA) : 0.0f;   // A = -exp(A_log)
        A2[j] = Av[j] * kLog2e;                            // A*log2(e)
        iA[j] = ok ? -expf(-al) : 0.0f;                    // 1/A
        if constexpr (PASS == 0) h[j] = (ok && p.h0) ? p.h0[(b * p.Dm + d) * p.N + n] : 0.0f;
        if constexpr (PASS == 1) h[j] = 0.0f;
        if constexpr (PASS == 3) h[j] = ok ? p.h_in[((b * p.nseg + seg) * p.Dm + d) * p.N + n] : 0.0f;
    }
    // per-element constants of the (t, d) elements this thread stages/reduces
    float biasv[EPT], Dv[EPT];
    bool cval[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int c = (tid + kThreads * i) % CW;
        const bool ok = d0 + c < p.Dm;
        cval[i] = ok;
        biasv[i] = (ok && p.dt_bias) ? p.dt_bias[d0 + c] : 0.0f;
        Dv[i] = (ok && p.D) ? p.D[d0 + c] : 0.0f;
    }
    // fused form: conv taps (zero past K), conv bias, and the carried inputs at
    // times -3, -2, -1 (zero before the state's K-1 steps)
    float cw[FUSE ? EPT : 1][kMaxConv], cb[FUSE ? EPT : 1], cs[FUSE ? EPT : 1][kMaxConv - 1];
    if constexpr (FUSE) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int c = (tid + kThreads * i) % CW;
            const bool ok = cval[i];
            const int64_t dd = d0 + c;
#pragma unroll
            for (int kk = 0; kk < kMaxConv; ++kk) cw[i][kk] = (ok && kk < p.K) ? p.conv_w[dd * p.K + kk] : 0.0f;
            cb[i] = (ok && p.conv_b) ? p.conv_b[dd] : 0.0f;
#pragma unroll
            for (int m = 0; m < kMaxConv - 1; ++m) {
                const int tt = m - (kMaxConv - 1);                 // time -3, -2, -1
                const bool in = ok && p.conv_state && tt >= -(p.K - 1);
                cs[i][m] = in ? p.conv_state[(b * p.Dm + dd) * (p.K - 1) + (p.K - 1) + tt] : 0.0f;
            }
        }
    }
    Ptrs<TIN, G, SPL> q;
    {
        const TIN *u = static_cast<const TIN *>(p.u);
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + kThreads * i;
            const int tl = e / CW, c = e % CW;
            const int64_t dd = min(d0 + c, p.Dm - 1);
            const int64_t off = (b * p.L + T0 + tl) * p.Dm + dd;     // time step tl of tile 0
            q.dt[i] = p.dt + off;
            q.u[i] = u + off;
            q.z[i] = (FUSE && p.z) ? static_cast<const TIN *>(p.z) + off : u + off;
            q.y[i] = p.y + (b * p.L + T0 + tl) * p.Dm + d0 + c;
        }
#pragma unroll
        for (int j = 0; j < SPL; ++j) q.nidx[j] = (int)min((int64_t)g * SPL + j, p.N - 1);
        const int64_t off = (b * p.L + T0 + k) * p.N;
        q.B = static_cast<const TIN *>(p.B) + off;
        q.C = static_cast<const TIN *>(p.C) + off;
    }
    const int64_t ntiles = (Lk + kT - 1) / kT;
    double dsum_acc = 0.0;   // PASS 1: this thread's sum of delta (one channel per thread)
    // Two register sets alternate between even and odd tiles, so that loads in
    // flight are never copied (a copy would force a wait on them).  The set of
    // tile k is loaded while tile k-2 is scanned; its dt/u are staged to LDS
    // while tile k-1 is scanned and its B/C are used when tile k is scanned.
    Raw<TIN, G, SPL, FUSE> RA, RB;
    float du_prev[EPT], du_cur[EPT];
    float gate_prev[FUSE ? EPT : 1], gate_cur[FUSE ? EPT : 1];   // SiLU(z), fused form

    auto stage = [&](int buf, int64_t t0, const Raw<TIN, G, SPL, FUSE> &R, auto chkTag) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + kThreads * i;
            const int tl = e / CW, c = e % CW;
            bool ok = cval[i];
            if constexpr (decltype(chkTag)::value) ok = ok && (t0 + tl < Lk);
            const float dl = ok ? softplus(R.dt[i] + biasv[i]) : 0.0f;
            if constexpr (PASS == 1) dsum_acc += (double)dl;
            float uu;
            if constexpr (FUSE) {
                float xk[kMaxConv] = {R.u[i], R.f.xh[i][0], R.f.xh[i][1], R.f.xh[i][2]};
                if constexpr (decltype(chkTag)::value) {
                    // steps before the sequence come from the carried state
#pragma unroll
                    for (int kk = 1; kk < kMaxConv; ++kk) {
                        const int64_t tt = t0 + tl - kk;
                        xk[kk] = tt == -1 ? cs[i][2] : tt == -2 ? cs[i][1] : tt == -3 ? cs[i][0] : xk[kk];
                    }
                }
                float pre = cb[i];
#pragma unroll
                for (int kk = 0; kk < kMaxConv; ++kk) pre = fmaf(cw[i][kk], xk[kk], pre);
                uu = ok ? silu_f(pre) : 0.0f;
                gate_cur[i] = p.z ? silu_f(R.f.z[i]) : 1.0f;
                if (p.u_out && ok) p.u_out[(b * p.L + t0 + tl) * p.Dm + d0 + c] = uu;
            } else {
                uu = ok ? R.u[i] : 0.0f;
            }
            sD[buf][c][tl] = dl;
            sU[buf][c][tl] = uu;
            du_cur[i] = Dv[i] * uu;
        }
    };

    auto compute = [&](int buf, const Raw<TIN, G, SPL, FUSE> &R) __attribute__((always_inline)) {
        float Bm[SPL], Cm[SPL];          // this tile's B, C (state-padding lanes zeroed)
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            Bm[j] = nval[j] ? R.B[j] : 0.0f;
            Cm[j] = nval[j] ? R.C[j] : 0.0f;
        }
        float yp[kT];
        static_for<0, kT / 4>([&](auto qi) __attribute__((always_inline)) {
            constexpr int q = decltype(qi)::value;
            const float4 dq = *reinterpret_cast<const float4 *>(&sD[buf][cl][4 * q]);
            const float4 uq = *reinterpret_cast<const float4 *>(&sU[buf][cl][4 * q]);
            const float dl4[4] = {dq.x, dq.y, dq.z, dq.w};
            const float uu4[4] = {uq.x, uq.y, uq.z, uq.w};
            static_for<0, 4>([&](auto ii) __attribute__((always_inline)) {
                constexpr int i = decltype(ii)::value;
                constexpr int t = 4 * q + i;
                const float dl = dl4[i], uu = uu4[i];
                float ys = 0.0f;
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const Zoh zh = zoh_exact(dl, Av[j], A2[j], iA[j]);   // Abar, (Abar - 1)/A
                    const float beta = MODE == 0 ? zh.beta : MODE == 1 ? dl : 1.0f;
                    const float bu = row_bcast<t>(Bm[j]) * uu;   // B[t, n] * u[t, d]
                    h[j] = hold_step<MODE>(h[j], zh.ab, Av[j], beta, bu);
                    if constexpr (YOUT) {
                        if (j == 0) ys = row_bcast<t>(Cm[j]) * h[j];
                        else ys = fmaf(row_bcast<t>(Cm[j]), h[j], ys);
                    }
                }
                yp[t] = ys;
            });
            if constexpr (YOUT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sY[buf][g][(4 * q + i) * CW + cl] = yp[4 * q + i];
            }
        });
    };

    auto reduce = [&](int buf, int64_t t0, auto chkTag) __attribute__((always_inline)) {
        if constexpr (!YOUT) return;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + kThreads * i;
            const int tl = e / CW, c = e % CW;
            float s = du_prev[i];
#pragma unroll
            for (int gg = 0; gg < G; ++gg) s += sY[buf][gg][tl * CW + c];
            if constexpr (FUSE) s *= gate_prev[i];
            bool ok = cval[i];
            if constexpr (decltype(chkTag)::value) ok = ok && (t0 + tl < Lk);
            if (ok) q.y[i][t0 * p.Dm] = s;
        }
    };

    // One tile: scan tile kt (its B/C in Rk), reduce tile kt-1, stage tile kt+1
    // (its dt/u in Rn), start loading tile kt+2 into Rk.  The steady-state body
    // is branch-free so that the loads stay in flight across iterations; the
    // first tile and the last few go through the checked body.
    auto shift = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) du_prev[i] = du_cur[i];
        if constexpr (FUSE) {
#pragma unroll
            for (int i = 0; i < EPT; ++i) gate_prev[i] = gate_cur[i];
        }
    };
    // SAVE: the state entering tile kt, before the tile is scanned
    auto save = [&](int64_t kt) __attribute__((always_inline)) {
        if constexpr (SAVE) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const int64_t n = (int64_t)g * SPL + j;
                if (dok && n < p.N) p.ck[((b * ntiles + kt) * p.Dm + d) * p.N + n] = h[j];
            }
        }
    };
    auto body_full = [&](int64_t kt, Raw<TIN, G, SPL, FUSE> &Rk, const Raw<TIN, G, SPL, FUSE> &Rn)
        __attribute__((always_inline)) {
        const int buf = (int)(kt & 1);
        save(kt);
        compute(buf, Rk);
        reduce(buf ^ 1, (kt - 1) * kT, std::false_type{});
        shift();
        stage(buf ^ 1, (kt + 1) * kT, Rn, std::false_type{});
        load_raw<false, YOUT>(Rk, q, p, Lk, (kt + 2) * kT, tid, k);
        __syncthreads();
    };
    auto body_checked = [&](int64_t kt, Raw<TIN, G, SPL, FUSE> &Rk, const Raw<TIN, G, SPL, FUSE> &Rn)
        __attribute__((always_inline)) {
        const int buf = (int)(kt & 1);
        save(kt);
        compute(buf, Rk);
        if (kt >= 1) reduce(buf ^ 1, (kt - 1) * kT, std::true_type{});
        shift();
        if (kt + 1 < ntiles) stage(buf ^ 1, (kt + 1) * kT, Rn, std::true_type{});
        if (kt + 2 < ntiles) load_raw<true, YOUT>(Rk, q, p, Lk, (kt + 2) * kT, tid, k);
        __syncthreads();
    };
    // The unchecked body of tile kt loads tile kt+2, so a pair (kt, kt+1) of
    // unchecked bodies needs tiles up to kt+3 to lie wholly inside the sequence.
    const int64_t nfull = Lk / kT;
    auto run = [&]() __attribute__((always_inline)) {
        int64_t kt = 0;
        if (ntiles >= 4) {
            body_checked(0, RA, RB);
            for (kt = 1; kt + 4 <= nfull; kt += 2) {   // tiles kt (set RB) and kt+1 (set RA)
                body_full(kt, RB, RA);
                body_full(kt + 1, RA, RB);
            }
        }
        for (; kt < ntiles; ++kt) {
            if (kt & 1) body_checked(kt, RB, RA);
            else body_checked(kt, RA, RB);
        }
    };

    load_raw<true, YOUT>(RA, q, p, Lk, 0, tid, k);
    if (ntiles > 1) load_raw<true, YOUT>(RB, q, p, Lk, kT, tid, k);
    stage(0, 0, RA, std::true_type{});
    __syncthreads();
    run();
    reduce((int)((ntiles - 1) & 1), (ntiles - 1) * kT, std::true_type{});

    if constexpr (PASS == 1) {
        // the segment's local state, and its sum of delta: the G threads of a
        // channel (tid = c + CW r) add their partial sums in a fixed order
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const int64_t n = (int64_t)g * SPL + j;
            if (dok && n < p.N) p.h_loc[((b * (p.nseg - 1) + seg) * p.Dm + d) * p.N + n] = h[j];
        }
        double *sS = reinterpret_cast<double *>(&sY[0][0][0]);   // sY is unused in this pass
        sS[tid] = dsum_acc;
        __syncthreads();
        if (tid < CW && d0 + tid < p.Dm) {
            double sacc = 0.0;
#pragma unroll
            for (int r = 0; r < G; ++r) sacc += sS[r * CW + tid];
            p.dsum[(b * (p.nseg - 1) + seg) * p.Dm + d0 + tid] = sacc;
        }
    } else if (p.h_final && (PASS == 0 || seg == p.nseg - 1)) {
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const int64_t n = (int64_t)g * SPL + j;
            if (dok && n < p.N) p.h_final[(b * p.Dm + d) * p.N + n] = h[j];
        }
    }
}

template <typename TIN, int G, int SPL, int MODE, bool FUSE, bool SAVE = false, int PASS = 0>
hipError_t launch_t(const S6Kp &kp, hipStream_t s) {
    constexpr int CW = kThreads / G;
    S6Kp p = kp;
    p.n_cblk = (p.Dm + CW - 1) / CW;
    const int64_t nseg_run = PASS == 0 ? 1 : PASS == 1 ? p.nseg - 1 : p.nseg;   // segments in this launch
    const int64_t nblk = p.batch * p.n_cblk * nseg_run;
    hipLaunchKernelGGL((s6_scan_kernel<TIN, G, SPL, MODE, FUSE, SAVE, PASS>), dim3((unsigned)nblk), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename TIN, int G, int SPL, bool FUSE, bool SAVE = false, int PASS = 0>
hipError_t launch_mode(const S6Kp &kp, int mode, hipStream_t s) {
    if (mode == 0) return launch_t<TIN, G, SPL, 0, FUSE, SAVE, PASS>(kp, s);
    if (mode == 1) return launch_t<TIN, G, SPL, 1, FUSE, SAVE, PASS>(kp, s);
    return launch_t<TIN, G, SPL, 2, FUSE, SAVE, PASS>(kp, s);
}

// the SAVE form, for the state sizes the S6 backward takes (N <= 16)
template <typename TIN>
hipError_t launch_shape_save(const S6Kp &kp, int mode, hipStream_t s) {
    const int64_t N = kp.N;
    if (N <= 1) return launch_mode<TIN, 1, 1, false, true>(kp, mode, s);
    if (N <= 2) return launch_mode<TIN, 2, 1, false, true>(kp, mode, s);
    if (N <= 4) return launch_mode<TIN, 4, 1, false, true>(kp, mode, s);
    if (N <= 8) return launch_mode<TIN, 8, 1, false, true>(kp, mode, s);
    return launch_mode<TIN, 16, 1, false, true>(kp, mode, s);
}

// the segmented passes, for the state sizes the segmented plan takes (N <= 16)
template <typename TIN, int PASS>
hipError_t launch_shape_seg(const S6Kp &kp, int mode, hipStream_t s) {
    const int64_t N = kp.N;
    if (N <= 1) return launch_mode<TIN, 1, 1, false, false, PASS>(kp, mode, s);
    if (N <= 2) return launch_mode<TIN, 2, 1, false, false, PASS>(kp, mode, s);
    if (N <= 4) return launch_mode<TIN, 4, 1, false, false, PASS>(kp, mode, s);
    if (N <= 8) return launch_mode<TIN, 8, 1, false, false, PASS>(kp, mode, s);
    return launch_mode<TIN, 16, 1, false, false, PASS>(kp, mode, s);
}

template <typename TIN, bool FUSE>
hipError_t launch_shape(const S6Kp &kp, int mode, hipStream_t s) {
    const int64_t N = kp.N;
    if (N <= 1) return launch_mode<TIN, 1, 1, FUSE>(kp, mode, s);
    if (N <= 2) return launch_mode<TIN, 2, 1, FUSE>(kp, mode, s);
    if (N <= 4) return launch_mode<TIN, 4, 1, FUSE>(kp, mode, s);
    if (N <= 8) return launch_mode<TIN, 8, 1, FUSE>(kp, mode, s);
    if (N <= 16) return launch_mode<TIN, 16, 1, FUSE>(kp, mode, s);
    if (N <= 32) return launch_mode<TIN, 16, 2, FUSE>(kp, mode, s);
    if (N <= 64) return launch_mode<TIN, 16, 4, FUSE>(kp, mode, s);
    if (N <= 128) return launch_mode<TIN, 16, 8, FUSE>(kp, mode, s);
    return launch_mode<TIN, 16, 16, FUSE>(kp, mode, s);
}

}  // namespace
}  // namespace ssm
