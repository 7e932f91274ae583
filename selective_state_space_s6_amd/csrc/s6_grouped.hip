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
};

// one tile's loads of one lane: B, C of its states at the tile's 16 steps, and
// dt, u of the step it stands for
template <int SPL>
struct GRaw {
    float B[kGT][SPL], C[kGT][SPL];
    float dt, u;
};

template <typename TIN, int SPL, int MODE>
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
    float A2[SPL], iA[SPL], h[SPL];
    bool small = false;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const int n = k + kGT * j;
        nval[j] = n < p.N;
        nidx[j] = nval[j] ? n : (int)p.N - 1;
        const bool ok = dval && nval[j];
        const float al = ok ? p.A_log[dd * p.N + n] : 0.0f;
        A2[j] = ok ? -expf(al) * kLog2e : 0.0f;          // A*log2(e), A = -exp(A_log)
        iA[j] = ok ? -expf(-al) : 0.0f;                  // 1/A
        h[j] = (ok && p.h0) ? p.h0[(b * p.Dm + d) * p.N + n] : 0.0f;
        small |= ok && (expf(al) < 0.125f);
    }
    // ZOH with |A| small: (e^z - 1)/A loses digits as z -> 0; such waves use a
    // series for phi1 when |z| < 1/16
    const bool acc_wave = (MODE == 0) && (__builtin_amdgcn_ballot_w64(small) != 0);
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

    auto compute = [&](const GRaw<SPL> &R, int64_t t0, auto accTag) __attribute__((always_inline)) {
        constexpr bool ACC = decltype(accTag)::value;
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
                const float x = dl * A2[j];
                const float ab = exp2_fast(x);                   // Abar = exp(delta*A)
                float beta;
                if constexpr (MODE == 0) {
                    beta = fmaf(ab, iA[j], -iA[j]);             // (Abar - 1)/A
                    if constexpr (ACC) {
                        const float z = x * kLn2;
                        if (fabsf(z) < 0.0625f) beta = dl * phi1_small(z);
                    }
                } else if constexpr (MODE == 1) {
                    beta = dl;
                } else {
                    beta = 1.0f;
                }
                h[j] = fmaf(ab, h[j], beta * (bm * uu));
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
        if (acc_wave) compute(RA, kt * kGT, std::true_type{});
        else compute(RA, kt * kGT, std::false_type{});
        if (kt + 2 < ntiles) load(RA, (kt + 2) * kGT);
        if (kt + 1 < ntiles) {
            if (acc_wave) compute(RB, (kt + 1) * kGT, std::true_type{});
            else compute(RB, (kt + 1) * kGT, std::false_type{});
            if (kt + 3 < ntiles) load(RB, (kt + 3) * kGT);
        }
    }
    if (p.h_final && dval) {
#pragma unroll
        for (int j = 0; j < SPL; ++j)
            if (nval[j]) p.h_final[(b * p.Dm + d) * p.N + k + kGT * j] = h[j];
    }
}

template <typename TIN, int SPL>
void launch_mode(const S6Gp &p, int mode, hipStream_t s) {
    const dim3 grid((unsigned)(p.batch * p.n_cblk)), block(kGThreads);
    if (mode == 0) hipLaunchKernelGGL((s6_grouped_kernel<TIN, SPL, 0>), grid, block, 0, s, p);
    else if (mode == 1) hipLaunchKernelGGL((s6_grouped_kernel<TIN, SPL, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((s6_grouped_kernel<TIN, SPL, 2>), grid, block, 0, s, p);
}

template <typename TIN>
void launch_spl(const S6Gp &p, int mode, hipStream_t s) {
    if (p.N <= kGT) launch_mode<TIN, 1>(p, mode, s);
    else launch_mode<TIN, 2>(p, mode, s);
}

}  // namespace

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

}  // namespace ssm
