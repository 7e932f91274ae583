// cssd_scan.hip -- complex-state SSD (Mamba-3 SISO style) forward scan, gfx950.
//
// Follows builderforce-memory-engine complex_ssd.ts (header comment,
// et_bbar_re/et_bbar_im, complex_ssd_forward): a complex diagonal state per
// (head channel p, complex state n), complex decay Abar_t = exp(delta_t*mu),
// complex input scale beta_t, output Re(C.h) + D x.  With a head-constant mu the
// decay from step s to step t is exp(mu (Lam_t - Lam_s)), Lam the running sum
// of delta, so the chunked decomposition of the real SSD applies with complex
// scalars.  Inside a 32-step chunk, with Lam counted from the chunk start and
// S the state entering the chunk:
//   y_t[p]  = Re(sum_n C_t[n] e^{mu Lam_t} S[p,n])                       (D5)
//           + sum_{s<=t} Re(G[t,s] e^{mu(Lam_t-Lam_s)} beta_s) x_s[p]   (D4)
//           + D x_t[p],   G[t,s] = sum_n C_t[n] B_s[n]
//   S'[p,n] = e^{mu Lam_end} S[p,n] + sum_s e^{mu(Lam_end-Lam_s)} beta_s B_s[n] x_s[p]   (D2, D3)
// Every decay is taken between two steps of one chunk (or from its start), so
// for the stable reading of A no exponent is positive.
//
// The multi-input multi-output form (builderforce-memory-engine mamba3_block.ts,
// module header item 2: R inputs and outputs per head and step sharing the
// state) runs through the same kernels: a step's R rows of x, y, B, C are
// consecutive and the kernels walk rows (see CssdKp::lgR).
//
// Layout of the work: as for the real SSD, the sequence of every (batch, head)
// is cut into segments (cssd_state_kernel: segment-local states and decays;
// cssd_pass_kernel: entering states; cssd_scan_kernel: outputs), and a work
// group holds one head with one wave per 16 head channels.  The complex state
// is stored as real pairs, k = 2n + (0 re, 1 im), and a wave keeps its
// 2Nc x 16 slice in fp32 MFMA accumulators (v_mfma_f32_16x16x4_f32).  Every
// contraction is a real fp32 GEMM on the matrix cores: complex products become
// sums over k of real products whose signs and re/im pairing are folded into
// the operands as they are read from LDS.  The 1e-4 tolerance of fp32 inputs
// rules out bf16 operands.  Running sums of delta are formed in double, so a
// rotation angle phi (Lam_t - Lam_s) carries only the rounding of its fp32
// difference.
#include "device_common.hpp"
#include "launchers.hpp"
#include <algorithm>
#include <type_traits>

namespace ssm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 32;              // steps per chunk
constexpr int kTargetWaves = 3072;  // enough resident waves to hide latency
constexpr int kMinSeg = 256;        // shortest segment worth a state round trip

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct cf { float re, im; };
__device__ __forceinline__ cf cmul(cf a, cf b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
__device__ __forceinline__ cf cexpf_(float re, float im) {
    float s, c;
    sincosf(im, &s, &c);
    const float m = expf(re);
    return {m * c, m * s};
}
// e^w - 1 without cancellation
__device__ __forceinline__ cf cexpm1f_(float re, float im) {
    float s, c;
    sincosf(im, &s, &c);
    const float sh = sinf(0.5f * im);
    return {expm1f(re) * c - 2.0f * sh * sh, expf(re) * s};
}
__device__ __forceinline__ cf cdiv(cf a, cf b) {
    const float den = b.re * b.re + b.im * b.im;
    return {(a.re * b.re + a.im * b.im) / den, (a.im * b.re - a.re * b.im) / den};
}

struct CssdKp {
    const float *x; const float *dt; const float *dt_bias; const float *A_log;
    const float *B; const float *C; const float *D; float *y;
    const float *h0; float *h_final;
    float *ws_state;    // (batch, H, nseg, P, 2 Nc): local, then entering, segment states
    float *ws_decay;    // (batch, H, nseg, 2): complex decay over a segment
    int64_t batch, L, H, P, Nc, G;
    int64_t Ls, nseg;   // segment length (a multiple of kT) and count
    uint32_t flags;
    // Multi-input multi-output form: R = 2^lgR inputs and outputs per head and
    // step, laid out as R consecutive rows of x, y, B, C per step.  The kernels
    // walk those rows as steps (L above counts them: L = R x steps); a row takes
    // dt of its step, the decay enters at the first row of a step only, every
    // row of a step has the step's input scale, and the causal mask compares
    // steps, so each output row of a step sees every input row of that step.
    int lgR;
};

// mu (the per-unit-delta complex rate) of head h for the selected reading
__device__ __forceinline__ cf head_mu(const CssdKp &p, int64_t h) {
    const float ell = p.A_log[2 * h], phi = p.A_log[2 * h + 1];
    const uint32_t am = p.flags & 0xCu;
    if (am == 0x4u) { float s, c; sincosf(phi, &s, &c); const float m = expf(ell); return {m * c, m * s}; }
    if (am == 0x8u) return {ell, phi};
    return {-expf(ell), phi};
}

__device__ __forceinline__ cf input_scale(const CssdKp &p, cf mu, float dl) {
    const uint32_t am = p.flags & 0xCu, bm = p.flags & 0x3u;
    if (am == 0x8u) {   // literal page kernel: (exp(delta*mu) - 1) * exp(-l - i*phi)
        const cf e1 = cexpm1f_(dl * mu.re, dl * mu.im);
        return cmul(e1, cexpf_(-mu.re, -mu.im));
    }
    if (bm == 1u) return {dl, 0.0f};
    if (bm == 2u) return {1.0f, 0.0f};
    if (mu.re == 0.0f && mu.im == 0.0f) return {dl, 0.0f};
    return cdiv(cexpm1f_(dl * mu.re, dl * mu.im), mu);   // (exp(delta*lambda) - 1)/lambda
}

// per-chunk scalars of one head, in LDS
struct CScal {
    double lam[kT];   // running sum of delta from the chunk start (inclusive)
    float2 bet[kT];   // beta_t
    float2 et[kT];    // e^{mu lam_t}
    float2 w[kT];     // e^{mu (lam_end - lam_s)} beta_s
    float2 E;         // e^{mu lam_end}
    double lend;      // lam_end
};

// Scalars of one chunk by one wave (lane = step within each 32-lane half; the
// upper half repeats the lower).  Steps past L have delta = beta = 0.
__device__ __forceinline__ void chunk_scalars(CScal &sc, const CssdKp &p, cf mu, double bias, float dtv,
                                              bool valid, int lane) {
    double dl = 0.0;
    cf be{0.0f, 0.0f};
    if (valid) {
        const double xv = (double)dtv + bias;
        dl = xv > 0.0 ? xv + log1p(exp(-xv)) : log1p(exp(xv));   // softplus
        be = input_scale(p, mu, (float)dl);
    }
    double v = (lane & ((1 << p.lgR) - 1)) == 0 ? dl : 0.0;   // the decay: once per step
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
        const double o = __shfl_up(v, off, 32);
        if ((lane & 31) >= off) v += o;
    }
    const double lend = __shfl(v, 31, 32);
    if (lane < kT) {
        const float lt = (float)v, lr = (float)(lend - v);
        const cf e = cexpf_(mu.re * lt, mu.im * lt);
        const cf w = cmul(cexpf_(mu.re * lr, mu.im * lr), be);
        sc.lam[lane] = v;
        sc.bet[lane] = make_float2(be.re, be.im);
        sc.et[lane] = make_float2(e.re, e.im);
        sc.w[lane] = make_float2(w.re, w.im);
    }
    if (lane == 0) {
        const float le = (float)lend;
        const cf E = cexpf_(mu.re * le, mu.im * le);
        sc.E = make_float2(E.re, E.im);
        sc.lend = lend;
    }
}

// Register and LDS staging of one chunk of x, B (and C), dt for a work group of
// NW waves holding head (b, h).  Rows are fp32; tiles have a padded pitch of
// KC + 4 (B, C) and P + 4 (x) floats.  Loads are unconditional so they stay in
// flight across a chunk; a chunk that crosses L clamps its step index into the
// tensors (rows past L never contribute: their delta and beta are 0 and their
// outputs are not stored).
template <int KC, int NW, bool WITH_C>
struct Stager {
    static constexpr int NTHR = 64 * NW;
    static constexpr int P = 16 * NW;
    static constexpr int CP = KC + 4;
    static constexpr int XP = P + 4;
    static constexpr int LDN = KC / 4;                          // 16-byte pieces per B/C row
    static constexpr int NBC = kT * LDN;                        // pieces per B (C) tile
    static constexpr int PBC = (NBC + NTHR - 1) / NTHR;
    static constexpr int XPR = P / 4;
    static constexpr int NX = kT * XPR;
    static constexpr int PX = NX / NTHR;
    static_assert(NX % NTHR == 0, "x pieces must divide over the group");

    // clang vector types: arrays of HIP's float4 (a class holding a union) stayed in
    // per-lane scratch memory, which also forced a wait on each prefetch
    f32x4 rB[PBC], rC[PBC], rX[PX];
    float rdt;
    const float *Bb, *Cb, *Xb, *Db;
    uint32_t oBC[PBC], oX[PX];   // per-piece offsets (floats) at chunk row 0
    int rBC[PBC], rXr[PX];       // per-piece rows
    int lBC[PBC], lX[PX];        // per-piece LDS offsets
    bool vBC[PBC];
    int sD, lgR;
    int64_t rowBC, rowX, H, L;

    __device__ __forceinline__ void init(const CssdKp &p, int64_t b, int64_t h, int64_t g, int tid) {
        rowBC = p.G * p.Nc * 2;
        rowX = p.H * p.P;
        H = p.H;
        L = p.L;
        const int K = (int)(2 * p.Nc);
#pragma unroll
        for (int i = 0; i < PBC; ++i) {
            const int pc = tid + NTHR * i;
            vBC[i] = pc < NBC;
            const int pcc = min(pc, NBC - 1);
            const int r = pcc / LDN, c = (pcc % LDN) * 4;
            rBC[i] = r;
            oBC[i] = (uint32_t)(r * rowBC + min(c, K - 4));
            lBC[i] = r * CP + c;
        }
#pragma unroll
        for (int i = 0; i < PX; ++i) {
            const int pc = tid + NTHR * i;
            const int r = pc / XPR, c = (pc % XPR) * 4;
            rXr[i] = r;
            oX[i] = (uint32_t)(r * rowX + c);
            lX[i] = r * XP + c;
        }
        sD = tid & 31;
        Bb = p.B + (b * p.L * p.G + g) * p.Nc * 2;
        Cb = p.C + (b * p.L * p.G + g) * p.Nc * 2;
        Xb = p.x + (b * p.L * p.H + h) * p.P;
        Db = p.dt + b * (p.L >> p.lgR) * p.H + h;
        lgR = p.lgR;
    }
    __device__ __forceinline__ void load(int64_t t0) {
        const float *Bu = Bb + t0 * rowBC, *Cu = Cb + t0 * rowBC, *Xu = Xb + t0 * rowX;
        const float *Du = Db + (t0 >> lgR) * H;     // t0 is a multiple of kT, so of R
        if (t0 + kT <= L) {
#pragma unroll
            for (int i = 0; i < PBC; ++i) {
                rB[i] = *reinterpret_cast<const f32x4 *>(Bu + oBC[i]);
                if constexpr (WITH_C) rC[i] = *reinterpret_cast<const f32x4 *>(Cu + oBC[i]);
            }
#pragma unroll
            for (int i = 0; i < PX; ++i) rX[i] = *reinterpret_cast<const f32x4 *>(Xu + oX[i]);
            rdt = Du[(uint32_t)((sD >> lgR) * H)];
        } else {
            const int last = (int)(L - 1 - t0);   // last valid step of the chunk
#pragma unroll
            for (int i = 0; i < PBC; ++i) {
                const uint32_t o = oBC[i] - (uint32_t)((rBC[i] - min(rBC[i], last)) * rowBC);
                rB[i] = *reinterpret_cast<const f32x4 *>(Bu + o);
                if constexpr (WITH_C) rC[i] = *reinterpret_cast<const f32x4 *>(Cu + o);
            }
#pragma unroll
            for (int i = 0; i < PX; ++i) {
                const uint32_t o = oX[i] - (uint32_t)((rXr[i] - min(rXr[i], last)) * rowX);
                rX[i] = *reinterpret_cast<const f32x4 *>(Xu + o);
            }
            rdt = Du[(uint32_t)((min(sD, last) >> lgR) * H)];
        }
    }
    __device__ __forceinline__ void store(float *Bs, float *Cs, float *Xs) {
#pragma unroll
        for (int i = 0; i < PBC; ++i) {
            if (PBC * NTHR == NBC || vBC[i]) {
                *reinterpret_cast<f32x4 *>(&Bs[lBC[i]]) = rB[i];
                if constexpr (WITH_C) *reinterpret_cast<f32x4 *>(&Cs[lBC[i]]) = rC[i];
            }
        }
#pragma unroll
        for (int i = 0; i < PX; ++i) *reinterpret_cast<f32x4 *>(&Xs[lX[i]]) = rX[i];
    }
};

// S <- E S (complex, the (re, im) pairs of a state tile sit in registers (0,1)
// and (2,3) of one lane)
template <int NTK>
__device__ __forceinline__ void decay_state(f32x4 (&S)[NTK], float2 E, int K) {
#pragma unroll
    for (int kt = 0; kt < NTK; ++kt) {
        if (kt * 16 >= K) break;
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
            const float re = S[kt][j], im = S[kt][j + 1];
            S[kt][j] = E.x * re - E.y * im;
            S[kt][j + 1] = E.x * im + E.y * re;
        }
    }
}

// D2: S[k][p] += sum_s (w B)_r[s][k] x[s][p] for one wave's 16 channels.  The A
// operand (row k = kt*16 + lane%16, K slot s = sb*16 + 4*(lane/16) + m) is the
// real or imaginary part of w_s B_s[n], n = k/2, formed as it is read.
template <int NTK, int CP, int XP>
__device__ __forceinline__ void state_add(f32x4 (&S)[NTK], const float *Bs, const float *Xs, const CScal &sc,
                                          int p0, int K, int lane) {
    const int c16 = lane & 15, q = lane >> 4;
    const bool odd = c16 & 1;
    // the chunk's contribution is summed on its own and added once, so its
    // roundings are relative to it and not to the (larger) state
    f32x4 dS[NTK];
#pragma unroll
    for (int kt = 0; kt < NTK; ++kt) dS[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int s = sb * 16 + 4 * q + m;
            const float2 w = sc.w[s];
            // even k: Re(w b) = w.re b.re - w.im b.im ; odd k: Im(w b) = w.im b.re + w.re b.im
            const float al = odd ? w.y : w.x, be = odd ? w.x : -w.y;
            const float xv = Xs[s * XP + p0 + c16];
#pragma unroll
            for (int kt = 0; kt < NTK; ++kt) {
                if (kt * 16 >= K) break;
                const float2 b = *reinterpret_cast<const float2 *>(&Bs[s * CP + kt * 16 + (c16 & ~1)]);
                dS[kt] = mfma4(fmaf(al, b.x, be * b.y), xv, dS[kt]);
            }
        }
    }
#pragma unroll
    for (int kt = 0; kt < NTK; ++kt) {
        if (kt * 16 >= K) break;
        S[kt] += dS[kt];
    }
}

// work index -> (b, segment, h); heads of one (batch, segment) are consecutive
struct Work {
    int64_t b, k, h;
    __device__ __forceinline__ Work(int64_t work, int64_t H, int64_t nseg)
        : b(work / (H * nseg)), k((work / H) % nseg), h(work % H) {}
};

// e^{mu lam} for a long running sum lam (double): the phase is reduced in double
__device__ __forceinline__ float2 cexp_long(cf mu, double lam) {
    double ph = (double)mu.im * lam;
    ph -= 6.283185307179586 * rint(ph * 0.15915494309189535);
    const cf e = cexpf_((float)((double)mu.re * lam), (float)ph);
    return make_float2(e.re, e.im);
}

// ---- segment-local final states (zero start) and the segment decay; every
// segment but the last, all of whose chunks are whole
template <int KC, bool EXACT, int NW>
__global__ void __launch_bounds__(64 * NW)
cssd_state_kernel(CssdKp p) {
    using St = Stager<KC, NW, false>;
    constexpr int NTK = KC / 16;
    constexpr int CP = St::CP, XP = St::XP;
    __shared__ __attribute__((aligned(16))) float Bs[2][kT * CP];
    __shared__ __attribute__((aligned(16))) float Xs[2][kT * XP];
    __shared__ CScal scal[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, q = lane >> 4;
    const int64_t nseg1 = p.nseg - 1;
    const Work wk(xcd_swizzle(blockIdx.x, p.batch * nseg1 * p.H), p.H, nseg1);
    const int64_t g = wk.h * p.G / p.H;
    const int p0 = wid * 16;
    const int K = EXACT ? KC : (int)(2 * p.Nc);
    const cf mu = head_mu(p, wk.h);
    const double bias = p.dt_bias ? (double)p.dt_bias[wk.h] : 0.0;

    f32x4 S[NTK];
#pragma unroll
    for (int kt = 0; kt < NTK; ++kt) S[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    St st;
    st.init(p, wk.b, wk.h, g, tid);
    const int64_t tb = wk.k * p.Ls;
    const int64_t nchunks = p.Ls / kT;
    st.load(tb);
    st.store(Bs[0], nullptr, Xs[0]);
    if (wid == 0) chunk_scalars(scal[0], p, mu, bias, st.rdt, true, lane);
    if (nchunks > 1) st.load(tb + kT);
    __syncthreads();

    double lseg = 0.0;
    for (int64_t j = 0; j < nchunks; ++j) {
        const int buf = (int)(j & 1);
        const CScal &sc = scal[buf];
        lseg += sc.lend;
        decay_state<NTK>(S, sc.E, K);
        state_add<NTK, CP, XP>(S, Bs[buf], Xs[buf], sc, p0, K, lane);
        if (j + 1 < nchunks) {
            st.store(Bs[buf ^ 1], nullptr, Xs[buf ^ 1]);
            if (wid == 0) chunk_scalars(scal[buf ^ 1], p, mu, bias, st.rdt, true, lane);
            if (j + 2 < nchunks) st.load(tb + (j + 2) * kT);
        }
        __syncthreads();
    }

    const int64_t slot = (wk.b * p.H + wk.h) * p.nseg + wk.k;
#pragma unroll
    for (int kt = 0; kt < NTK; ++kt) {
        if (kt * 16 >= K) break;
        float *dst = p.ws_state + (slot * p.P + p0 + c16) * (2 * p.Nc) + kt * 16 + q * 4;
        *reinterpret_cast<float4 *>(dst) = make_float4(S[kt][0], S[kt][1], S[kt][2], S[kt][3]);
    }
    if (tid == 0) {
        const float2 d = cexp_long(mu, lseg);
        p.ws_decay[2 * slot] = d.x;
        p.ws_decay[2 * slot + 1] = d.y;
    }
}

// ---- D3 across segments: the state entering each segment, in place of the
// segment-local states.  One thread per 2 complex (p, n) of one (b, h).
__global__ void __launch_bounds__(256)
cssd_pass_kernel(CssdKp p) {
    const int64_t per = p.P * p.Nc / 2;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= p.batch * p.H * per) return;
    const int64_t bh = i / per, e = i % per;
    float4 S = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (p.h0) S = reinterpret_cast<const float4 *>(p.h0)[bh * per + e];
    float4 *ws = reinterpret_cast<float4 *>(p.ws_state) + bh * p.nseg * per + e;
    for (int64_t k = 0; k + 1 < p.nseg; ++k) {
        const float4 loc = ws[k * per];
        const float dr = p.ws_decay[2 * (bh * p.nseg + k)], di = p.ws_decay[2 * (bh * p.nseg + k) + 1];
        ws[k * per] = S;
        S = make_float4(dr * S.x - di * S.y + loc.x, dr * S.y + di * S.x + loc.y,
                        dr * S.z - di * S.w + loc.z, dr * S.w + di * S.z + loc.w);
    }
    ws[(p.nseg - 1) * per] = S;
}

// ---- outputs of one segment from the state entering it
template <int KC, bool EXACT, int NW>
__global__ void __launch_bounds__(64 * NW)
cssd_scan_kernel(CssdKp p) {
    using St = Stager<KC, NW, true>;
    constexpr int NTK = KC / 16;
    constexpr int CP = St::CP, XP = St::XP;
    __shared__ __attribute__((aligned(16))) float Bs[2][kT * CP];
    __shared__ __attribute__((aligned(16))) float Cs[2][kT * CP];
    __shared__ __attribute__((aligned(16))) float Xs[2][kT * XP];
    // the chunk's causal tiles of M[t][s] = Re(G[t,s] e^{mu(lam_t-lam_s)} beta_s) as
    // the A fragments of M X: tile tau = (s-tile, t-tile) (0,0), (0,1), (1,1)
    __shared__ __attribute__((aligned(16))) f32x4 Ms[3][64];
    __shared__ CScal scal[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, q = lane >> 4;
    const Work wk(xcd_swizzle(blockIdx.x, p.batch * p.nseg * p.H), p.H, p.nseg);
    const int64_t g = wk.h * p.G / p.H;
    const int p0 = wid * 16;
    const int K = EXACT ? KC : (int)(2 * p.Nc);
    const cf mu = head_mu(p, wk.h);
    const double bias = p.dt_bias ? (double)p.dt_bias[wk.h] : 0.0;
    const float csign = (p.flags & 0x10u) ? -1.0f : 1.0f;   // conj(C)
    const float Dh = p.D ? p.D[wk.h] : 0.0f;
    const int64_t rowX = p.H * p.P;
    float *Yg = p.y + (wk.b * p.L * p.H + wk.h) * p.P + p0;
    const uint32_t ylane = (uint32_t)(q * 4 * rowX + c16) * 4u;   // byte offset of the lane's element

    // state slice S_r[k][p], k = 2n + (re, im), p in this wave's 16 channels, in
    // the MFMA output layout: tile kt, lane (column p = c16, rows k = kt*16 + q*4 + v)
    const float *Sin = p.nseg > 1 ? p.ws_state + ((wk.b * p.H + wk.h) * p.nseg + wk.k) * p.P * 2 * p.Nc
                                  : (p.h0 ? p.h0 + (wk.b * p.H + wk.h) * p.P * 2 * p.Nc : nullptr);
    f32x4 S[NTK];
#pragma unroll
    for (int kt = 0; kt < NTK; ++kt) {
        S[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (Sin && kt * 16 < K) {
            const float4 v = *reinterpret_cast<const float4 *>(Sin + (p0 + c16) * 2 * p.Nc + kt * 16 + q * 4);
            S[kt] = f32x4{v.x, v.y, v.z, v.w};
        }
    }

    St st;
    st.init(p, wk.b, wk.h, g, tid);
    const int64_t tb = wk.k * p.Ls;
    const int64_t te = min(tb + p.Ls, p.L);
    const int64_t nchunks = (te - tb + kT - 1) / kT;
    st.load(tb);
    st.store(Bs[0], Cs[0], Xs[0]);
    if (wid == NW - 1) chunk_scalars(scal[0], p, mu, bias, st.rdt, tb + (lane & 31) < p.L, lane);
    if (nchunks > 1) st.load(tb + kT);
    __syncthreads();

    for (int64_t j = 0; j < nchunks; ++j) {
        const int buf = (int)(j & 1);
        const int64_t t0 = tb + j * kT;
        const float *B_ = Bs[buf], *C_ = Cs[buf], *X_ = Xs[buf];
        const CScal &sc = scal[buf];

        // D4, shared: G^T[s][t] (re and im) for the causal tile pairs, one per
        // wave (wave tau % NW).  Lane holds column t = tT*16 + c16, rows
        // s = sT*16 + q*4 + v.  K slot (q, m) of block kb is k = kb*16 + 4q + m.
        //   Re G = sum_n B_re C_re - B_im C_im,  Im G = sum_n B_re C_im + B_im C_re
        // (C_im -> -C_im for conj(C)).
#pragma unroll
        for (int tau = 0; tau < 3; ++tau) {
            if (tau % NW != wid) continue;
            const int sT = tau == 2 ? 1 : 0, tT = tau == 0 ? 0 : 1;
            f32x4 Gr{0.0f, 0.0f, 0.0f, 0.0f}, Gi{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < NTK; ++kb) {
                if (kb * 16 >= K) break;
                const float4 bq = *reinterpret_cast<const float4 *>(&B_[(sT * 16 + c16) * CP + kb * 16 + 4 * q]);
                const float4 cq = *reinterpret_cast<const float4 *>(&C_[(tT * 16 + c16) * CP + kb * 16 + 4 * q]);
                const float c1 = csign * cq.y, c3 = csign * cq.w;
                Gr = mfma4(bq.x, cq.x, Gr);
                Gr = mfma4(-bq.y, c1, Gr);
                Gr = mfma4(bq.z, cq.z, Gr);
                Gr = mfma4(-bq.w, c3, Gr);
                Gi = mfma4(bq.y, cq.x, Gi);
                Gi = mfma4(bq.x, c1, Gi);
                Gi = mfma4(bq.w, cq.z, Gi);
                Gi = mfma4(bq.z, c3, Gi);
            }
            const int t = tT * 16 + c16;
            const double lt = sc.lam[t];
            f32x4 mv;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int s = sT * 16 + 4 * q + v;
                float m = 0.0f;
                if ((s >> p.lgR) <= (t >> p.lgR)) {      // causal over steps
                    const float dl = (float)(lt - sc.lam[s]);
                    const float2 bs = sc.bet[s];
                    const cf f = cmul(cexpf_(mu.re * dl, mu.im * dl), cf{bs.x, bs.y});
                    m = Gr[v] * f.re - Gi[v] * f.im;
                }
                mv[v] = m;
            }
            Ms[tau][lane] = mv;
        }

        // D5: ys[tt] = sum_k Chat[t][k] S_r[k][p], Chat = (Re, -Im) of C_t[n] e^{mu lam_t};
        // two partial sums (even and odd state tiles) shorten the fp32 chains
        f32x4 ys[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            ys[tt][0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            ys[tt][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const float2 e = sc.et[tt * 16 + c16];
#pragma unroll
            for (int kt = 0; kt < NTK; ++kt) {
                if (kt * 16 >= K) break;
                const float4 cq = *reinterpret_cast<const float4 *>(&C_[(tt * 16 + c16) * CP + kt * 16 + 4 * q]);
                const float ci0 = csign * cq.y, ci1 = csign * cq.w;
                f32x4 &a = ys[tt][kt & 1];
                a = mfma4(cq.x * e.x - ci0 * e.y, S[kt][0], a);
                a = mfma4(-(cq.x * e.y + ci0 * e.x), S[kt][1], a);
                a = mfma4(cq.z * e.x - ci1 * e.y, S[kt][2], a);
                a = mfma4(-(cq.z * e.y + ci1 * e.x), S[kt][3], a);
            }
        }

        __syncthreads();   // the shared M fragments are complete

        // D4: acc[tt] = sum_{s-tile <= tt} M X
        f32x4 acc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int tau = 0; tau < 3; ++tau) {
            const int sT = tau == 2 ? 1 : 0, tT = tau == 0 ? 0 : 1;
            const f32x4 mv = Ms[tau][lane];
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[tT] = mfma4(mv[m], X_[(sT * 16 + 4 * q + m) * XP + p0 + c16], acc[tT]);
        }

        // skip term and store: lane (column p0 + c16, rows t = tt*16 + q*4 + v)
        float yv[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                yv[tt][v] = fmaf(Dh, X_[(tt * 16 + 4 * q + v) * XP + p0 + c16],
                                 (ys[tt][0][v] + ys[tt][1][v]) + acc[tt][v]);
        if (t0 + kT <= te) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    *reinterpret_cast<float *>(reinterpret_cast<char *>(Yg + (t0 + tt * 16 + v) * rowX) + ylane) =
                        yv[tt][v];
        } else {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (t0 + tt * 16 + q * 4 + v < te)
                        *reinterpret_cast<float *>(reinterpret_cast<char *>(Yg + (t0 + tt * 16 + v) * rowX) + ylane) =
                            yv[tt][v];
        }

        // D2 + D3
        decay_state<NTK>(S, sc.E, K);
        state_add<NTK, CP, XP>(S, B_, X_, sc, p0, K, lane);

        // stage chunk j+1, start loading chunk j+2
        if (j + 1 < nchunks) {
            st.store(Bs[buf ^ 1], Cs[buf ^ 1], Xs[buf ^ 1]);
            if (wid == NW - 1)   // the wave with no decay-mask tile (or the least)
                chunk_scalars(scal[buf ^ 1], p, mu, bias, st.rdt, t0 + kT + (lane & 31) < p.L, lane);
            if (j + 2 < nchunks) st.load(t0 + 2 * kT);
        }
        __syncthreads();
    }

    if (p.h_final && wk.k == p.nseg - 1) {
#pragma unroll
        for (int kt = 0; kt < NTK; ++kt) {
            if (kt * 16 >= K) break;
            float *dst = p.h_final + ((wk.b * p.H + wk.h) * p.P + p0 + c16) * 2 * p.Nc + kt * 16 + q * 4;
            *reinterpret_cast<float4 *>(dst) = make_float4(S[kt][0], S[kt][1], S[kt][2], S[kt][3]);
        }
    }
}

struct Plan {
    int64_t nseg, Ls;
};
Plan plan(int64_t batch, int64_t L, int64_t H, int64_t P) {
    const int64_t waves = batch * H * (P / 16);
    int64_t nseg = (kTargetWaves + waves - 1) / waves;
    nseg = std::max<int64_t>(1, std::min<int64_t>(nseg, L / kMinSeg));
    const int64_t Ls = ((L + nseg - 1) / nseg + kT - 1) / kT * kT;
    return Plan{(L + Ls - 1) / Ls, Ls};
}
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

template <int KC, bool EXACT, int NW>
void launch_all(const CssdKp &p, hipStream_t stream) {
    if (p.nseg > 1) {
        const int64_t n1 = p.batch * (p.nseg - 1) * p.H;
        hipLaunchKernelGGL((cssd_state_kernel<KC, EXACT, NW>), dim3((unsigned)n1), dim3(64 * NW), 0, stream, p);
        const int64_t nt = p.batch * p.H * p.P * p.Nc / 2;
        hipLaunchKernelGGL(cssd_pass_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, stream, p);
    }
    const int64_t n = p.batch * p.nseg * p.H;
    hipLaunchKernelGGL((cssd_scan_kernel<KC, EXACT, NW>), dim3((unsigned)n), dim3(64 * NW), 0, stream, p);
}

template <int NW>
void launch_k(const CssdKp &p, hipStream_t stream) {
    const int64_t K = 2 * p.Nc;
    if (K == 16) return launch_all<16, true, NW>(p, stream);
    if (K == 32) return launch_all<32, true, NW>(p, stream);
    if (K == 64) return launch_all<64, true, NW>(p, stream);
    if (K < 64) return launch_all<64, false, NW>(p, stream);
    if (K == 128) return launch_all<128, true, NW>(p, stream);
    launch_all<128, false, NW>(p, stream);
}

}  // namespace

size_t cssd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t n_complex,
                            int64_t) {
    const Plan pl = plan(batch, L, nheads, headdim);
    if (pl.nseg <= 1) return 0;
    return align256((size_t)(batch * nheads * pl.nseg * headdim * n_complex * 2) * sizeof(float)) +
           (size_t)(batch * nheads * pl.nseg * 2) * sizeof(float);
}

hipError_t launch_cssd(const CssdArgs &a, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "cssd_scan_kernel";
    CssdKp p{};
    p.x = a.x; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C;
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L * a.rank; p.H = a.nheads; p.P = a.headdim; p.Nc = a.n_complex; p.G = a.ngroups;
    p.flags = a.flags;
    p.lgR = 0;
    while ((int64_t(1) << p.lgR) < a.rank) ++p.lgR;
    const Plan pl = plan(p.batch, p.L, p.H, p.P);
    p.nseg = pl.nseg;
    p.Ls = pl.Ls;
    if (p.nseg > 1) {
        p.ws_state = static_cast<float *>(a.workspace);
        p.ws_decay = reinterpret_cast<float *>(
            static_cast<char *>(a.workspace) +
            align256((size_t)(p.batch * p.H * p.nseg * p.P * p.Nc * 2) * sizeof(float)));
    }
    if (p.P == 32) launch_k<2>(p, stream);
    else if (p.P == 64) launch_k<4>(p, stream);
    else launch_k<8>(p, stream);
    return hipGetLastError();
}

}  // namespace ssm
