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
// Layout of the work: cssd_prep_kernel first takes, once per (batch, chunk,
// head), everything that does not depend on the head channel: the chunk's
// running sums of delta, input scales and decays (a record of w_s, e^{mu Lam_t}
// and the chunk decay), and the causal tiles of M[t][s] = Re(G[t,s]
// e^{mu(Lam_t-Lam_s)} beta_s), with G = C.B^T formed once per group of heads.
// Then, as for the real SSD, the sequence of every (batch, head) is cut into
// segments (cssd_state_kernel: segment-local states and decays;
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
// word 3 of a raw buffer resource on gfx9-family chips (gfx950 included): 32-bit data
// format, no swizzle, no index stride; with stride 0 a store at or past the record count
// is dropped
constexpr int kBufWord3 = 0x00020000;

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

// per-(batch, head, chunk) record of the chunk scalars the state and output
// passes use, written by cssd_prep_kernel
struct CRec {
    float2 w[kT];     // e^{mu (lam_end - lam_s)} beta_s
    float2 et[kT];    // e^{mu lam_t}
    float2 E;         // e^{mu lam_end}
    double lend;      // lam_end
};
static_assert(sizeof(CRec) == 33 * 16, "a record is 33 16-byte pieces");

struct CssdKp {
    const float *x; const float *dt; const float *dt_bias; const float *A_log;
    const float *B; const float *C; const float *D; float *y;
    const float *h0; float *h_final;
    float *ws_state;    // (batch, H, nseg, P, 2 Nc): local, then entering, segment states
    float *ws_decay;    // (batch, H, nseg, 2): complex decay over a segment
    CRec *rec;          // (batch, H, nck) chunk records
    f32x4 *mtile;       // (batch, H, nck, 3, 64): the causal M tiles as MFMA A fragments
    int64_t batch, L, H, P, Nc, G;
    int64_t Ls, nseg;   // segment length (a multiple of kT) and count
    int64_t nck;        // chunks of the whole sequence
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

// Scalars of one chunk of one head by one 32-lane half of a wave (step
// lane & 31; the two halves may hold two heads, each with its own sc, mu,
// bias).  Steps past L have delta = beta = 0.
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
    const int t = lane & 31;
    {
        const float lt = (float)v, lr = (float)(lend - v);
        const cf e = cexpf_(mu.re * lt, mu.im * lt);
        const cf w = cmul(cexpf_(mu.re * lr, mu.im * lr), be);
        sc.lam[t] = v;
        sc.bet[t] = make_float2(be.re, be.im);
        sc.et[t] = make_float2(e.re, e.im);
        sc.w[t] = make_float2(w.re, w.im);
    }
    if (t == 0) {
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
    float2 rW[PBC], rE[PBC];     // w and e^{mu lam} of each piece's step, from the chunk record
    const float *Bb, *Cb, *Xb;
    const CRec *Rb;
    uint32_t oBC[PBC], oX[PX];   // per-piece offsets (floats) at chunk row 0
    int rBC[PBC], rXr[PX];       // per-piece rows
    int lBC[PBC], lX[PX];        // per-piece LDS offsets
    bool vBC[PBC];
    int64_t rowBC, rowX, L;

    __device__ __forceinline__ void init(const CssdKp &p, int64_t b, int64_t h, int64_t g, int tid) {
        rowBC = p.G * p.Nc * 2;
        rowX = p.H * p.P;
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
        Bb = p.B + (b * p.L * p.G + g) * p.Nc * 2;
        Cb = p.C + (b * p.L * p.G + g) * p.Nc * 2;
        Xb = p.x + (b * p.L * p.H + h) * p.P;
        Rb = p.rec + (b * p.H + h) * p.nck;
    }
    // chunk t0 / kT: its rows and, per B/C piece, its step's scalars
    __device__ __forceinline__ void load(int64_t t0) {
        const float *Bu = Bb + t0 * rowBC, *Cu = Cb + t0 * rowBC, *Xu = Xb + t0 * rowX;
        const CRec &rn = Rb[t0 / kT];
#pragma unroll
        for (int i = 0; i < PBC; ++i) {
            rW[i] = rn.w[rBC[i]];
            if constexpr (WITH_C) rE[i] = rn.et[rBC[i]];
        }
        if (t0 + kT <= L) {
#pragma unroll
            for (int i = 0; i < PBC; ++i) {
                rB[i] = *reinterpret_cast<const f32x4 *>(Bu + oBC[i]);
                if constexpr (WITH_C) rC[i] = *reinterpret_cast<const f32x4 *>(Cu + oBC[i]);
            }
#pragma unroll
            for (int i = 0; i < PX; ++i) rX[i] = *reinterpret_cast<const f32x4 *>(Xu + oX[i]);
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
        }
    }
    // The B and C tiles go to LDS as the operands every wave of the group
    // uses, formed once here from the chunk record's scalars (a row past L
    // has w = 0, and its output is not stored):
    //   B -> w_s B_s[n] as real pairs (Re, Im): the D2 operand;
    //   C -> C_t[n] e^{mu lam_t} as (Re, -Im): the D5 operand (conj(C) by csign).
    __device__ __forceinline__ void store(float *Bs, float *Cs, float *Xs, float csign) {
#pragma unroll
        for (int i = 0; i < PBC; ++i) {
            if (PBC * NTHR == NBC || vBC[i]) {
                const float2 w = rW[i];
                const f32x4 b = rB[i];
                f32x4 wb;
                wb[0] = fmaf(w.x, b[0], -w.y * b[1]);   // Re(w b) = w.re b.re - w.im b.im
                wb[1] = fmaf(w.y, b[0], w.x * b[1]);    // Im(w b) = w.im b.re + w.re b.im
                wb[2] = fmaf(w.x, b[2], -w.y * b[3]);
                wb[3] = fmaf(w.y, b[2], w.x * b[3]);
                *reinterpret_cast<f32x4 *>(&Bs[lBC[i]]) = wb;
                if constexpr (WITH_C) {
                    const float2 e = rE[i];
                    const f32x4 cq = rC[i];
                    const float ci0 = csign * cq[1], ci1 = csign * cq[3];
                    // the fused forms are written out, so the operand's rounding
                    // does not depend on the compiler's contraction choices
                    f32x4 ch;
                    ch[0] = fmaf(cq[0], e.x, -(ci0 * e.y));    // Re(C e)
                    ch[1] = -fmaf(cq[0], e.y, ci0 * e.x);      // -Im(C e)
                    ch[2] = fmaf(cq[2], e.x, -(ci1 * e.y));
                    ch[3] = -fmaf(cq[2], e.y, ci1 * e.x);
                    *reinterpret_cast<f32x4 *>(&Cs[lBC[i]]) = ch;
                }
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
// operand (row k = kt*16 + lane%16, K slot s = sb*16 + 4*(lane/16) + m) is
// entry k of w_s B_s as real pairs, formed when the tile was staged.
template <int NTK, int CP, int XP>
__device__ __forceinline__ void state_add(f32x4 (&S)[NTK], const float *WB, const float *Xs, int p0, int K,
                                          int lane) {
    const int c16 = lane & 15, q = lane >> 4;
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
            const float xv = Xs[s * XP + p0 + c16];
#pragma unroll
            for (int kt = 0; kt < NTK; ++kt) {
                if (kt * 16 >= K) break;
                dS[kt] = mfma4(WB[s * CP + kt * 16 + c16], xv, dS[kt]);
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

// ---- chunk records and M tiles: two heads per wave (one per 32-lane half for
// the chunk scalars), eight heads of one group per work group.  Waves 0-2
// first form G = C.B^T over the chunk's causal tile pairs (tau = (s-tile,
// t-tile) = (0,0), (0,1), (1,1)), which every head of the group shares; then
// every wave takes its heads' chunk scalars and applies each head's decay and
// input scale to G.
template <int KC, bool EXACT>
__global__ void __launch_bounds__(256)
cssd_prep_kernel(CssdKp p) {
    constexpr int NTK = KC / 16;
    __shared__ f32x4 Gs[3][2][64];   // Re G^T and Im G^T tiles, lane-major as MFMA outputs
    __shared__ CScal scal[8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, q = lane >> 4;
    const int64_t Hg = p.H / p.G, nq = (Hg + 7) / 8;
    int64_t r = xcd_swizzle(blockIdx.x, p.batch * p.nck * p.G * nq);   // the blocks of a group stay together
    const int64_t hq = r % nq;
    r /= nq;
    const int64_t g = r % p.G;
    r /= p.G;
    const int64_t c = r % p.nck, b = r / p.nck;
    const int64_t t0 = c * kT;
    const int last = (int)min<int64_t>(kT - 1, p.L - 1 - t0);   // last valid step of the chunk
    const int K = EXACT ? KC : (int)(2 * p.Nc);
    const float csign = (p.flags & 0x10u) ? -1.0f : 1.0f;   // conj(C)

    // G^T[s][t] (re and im) for tile pair tau = wid.  Lane holds column
    // t = tT*16 + c16, rows s = sT*16 + q*4 + v; K slot (q, m) of block kb is
    // k = kb*16 + 4q + m.
    //   Re G = sum_n B_re C_re - B_im C_im,  Im G = sum_n B_re C_im + B_im C_re
    // (C_im -> -C_im for conj(C)).  Rows past L repeat the last valid row.
    if (wid < 3) {
        const int sT = wid == 2 ? 1 : 0, tT = wid == 0 ? 0 : 1;
        const int64_t rowBC = p.G * p.Nc * 2;
        const float *Bg = p.B + ((b * p.L + t0) * p.G + g) * p.Nc * 2;
        const float *Cg = p.C + ((b * p.L + t0) * p.G + g) * p.Nc * 2;
        const float *Brow = Bg + min(sT * 16 + c16, last) * rowBC + 4 * q;
        const float *Crow = Cg + min(tT * 16 + c16, last) * rowBC + 4 * q;
        f32x4 Gr{0.0f, 0.0f, 0.0f, 0.0f}, Gi{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < NTK; ++kb) {
            if (kb * 16 >= K) break;
            const float4 bq = *reinterpret_cast<const float4 *>(Brow + kb * 16);
            const float4 cq = *reinterpret_cast<const float4 *>(Crow + kb * 16);
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
        Gs[wid][0][lane] = Gr;
        Gs[wid][1][lane] = Gi;
    }

    // chunk scalars: half hf of the wave takes head hq*8 + 2*wid + hf of the group
    const int64_t hbase = hq * 8 + 2 * wid;   // within the group
    if (hbase < Hg) {                          // uniform over the wave
        const int hf = lane >> 5;
        const bool hok = hbase + hf < Hg;
        const int64_t h = g * Hg + min<int64_t>(hbase + hf, Hg - 1);
        const double bias = p.dt_bias ? (double)p.dt_bias[h] : 0.0;
        const int64_t step = (t0 + min(lane & 31, last)) >> p.lgR;
        const float dtv = p.dt[(b * (p.L >> p.lgR) + step) * p.H + h];
        chunk_scalars(scal[2 * wid + hf], p, head_mu(p, h), bias, dtv, hok && t0 + (lane & 31) < p.L, lane);
    }
    __syncthreads();

    for (int hf = 0; hf < 2; ++hf) {
        if (hbase + hf >= Hg) break;   // uniform over the wave
        const int64_t h = g * Hg + hbase + hf;
        const cf mu = head_mu(p, h);
        const CScal &sc = scal[2 * wid + hf];

        // M tiles: M^T[s][t] = Re(G[t,s] e^{mu(lam_t-lam_s)} beta_s), causal over steps
        f32x4 *Mo = p.mtile + ((b * p.H + h) * p.nck + c) * 192 + lane;
#pragma unroll
        for (int tau = 0; tau < 3; ++tau) {
            const int sT = tau == 2 ? 1 : 0, tT = tau == 0 ? 0 : 1;
            const f32x4 Gr = Gs[tau][0][lane], Gi = Gs[tau][1][lane];
            const int t = tT * 16 + c16;
            const double lt = sc.lam[t];
            f32x4 mv;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int s = sT * 16 + 4 * q + v;
                float m = 0.0f;
                if ((s >> p.lgR) <= (t >> p.lgR)) {
                    const float dl = (float)(lt - sc.lam[s]);
                    const float2 bs = sc.bet[s];
                    const cf f = cmul(cexpf_(mu.re * dl, mu.im * dl), cf{bs.x, bs.y});
                    m = Gr[v] * f.re - Gi[v] * f.im;
                }
                mv[v] = m;
            }
            Mo[tau * 64] = mv;
        }

        CRec *R = p.rec + (b * p.H + h) * p.nck + c;
        if (lane < kT) {
            R->w[lane] = sc.w[lane];
            R->et[lane] = sc.et[lane];
        }
        if (lane == 0) {
            R->E = sc.E;
            R->lend = sc.lend;
        }
    }
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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, q = lane >> 4;
    const int64_t nseg1 = p.nseg - 1;
    const Work wk(xcd_swizzle(blockIdx.x, p.batch * nseg1 * p.H), p.H, nseg1);
    const int64_t g = wk.h * p.G / p.H;
    const int p0 = wid * 16;
    const int K = EXACT ? KC : (int)(2 * p.Nc);

    f32x4 S[NTK];
#pragma unroll
    for (int kt = 0; kt < NTK; ++kt) S[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    St st;
    st.init(p, wk.b, wk.h, g, tid);
    const int64_t tb = wk.k * p.Ls;
    const CRec *Rc = p.rec + (wk.b * p.H + wk.h) * p.nck + tb / kT;   // the segment's chunk records
    const int64_t nchunks = p.Ls / kT;
    st.load(tb);
    st.store(Bs[0], nullptr, Xs[0], 1.0f);
    if (nchunks > 1) st.load(tb + kT);
    __syncthreads();

    double lseg = 0.0;
    for (int64_t j = 0; j < nchunks; ++j) {
        const int buf = (int)(j & 1);
        lseg += Rc[j].lend;
        decay_state<NTK>(S, Rc[j].E, K);
        state_add<NTK, CP, XP>(S, Bs[buf], Xs[buf], p0, K, lane);
        if (j + 1 < nchunks) {
            st.store(Bs[buf ^ 1], nullptr, Xs[buf ^ 1], 1.0f);
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
        const float2 d = cexp_long(head_mu(p, wk.h), lseg);
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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, q = lane >> 4;
    const Work wk(xcd_swizzle(blockIdx.x, p.batch * p.nseg * p.H), p.H, p.nseg);
    const int64_t g = wk.h * p.G / p.H;
    const int p0 = wid * 16;
    const int K = EXACT ? KC : (int)(2 * p.Nc);
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
    const int64_t c0 = tb / kT;
    const int64_t nchunks = (te - tb + kT - 1) / kT;
    const CRec *Rc = p.rec + (wk.b * p.H + wk.h) * p.nck + c0;   // the segment's chunk records
    // the chunk's M fragments (tile tau at lane), read a chunk ahead
    const f32x4 *Mg = p.mtile + ((wk.b * p.H + wk.h) * p.nck + c0) * 192 + lane;
    f32x4 mnext[3];
#pragma unroll
    for (int tau = 0; tau < 3; ++tau) mnext[tau] = Mg[tau * 64];
    float2 Enext = Rc[0].E;   // the chunk's state decay, also read a chunk ahead
    st.load(tb);
    st.store(Bs[0], Cs[0], Xs[0], csign);
    if (nchunks > 1) st.load(tb + kT);
    __syncthreads();

    for (int64_t j = 0; j < nchunks; ++j) {
        const int buf = (int)(j & 1);
        const int64_t t0 = tb + j * kT;
        const float *B_ = Bs[buf], *C_ = Cs[buf], *X_ = Xs[buf];
        const float2 E = Enext;
        f32x4 mv[3];
#pragma unroll
        for (int tau = 0; tau < 3; ++tau) mv[tau] = mnext[tau];
        if (j + 1 < nchunks) {
#pragma unroll
            for (int tau = 0; tau < 3; ++tau) mnext[tau] = Mg[(j + 1) * 192 + tau * 64];
            Enext = Rc[j + 1].E;
        }
        // D5: ys[tt] = sum_k Chat[t][k] S_r[k][p], Chat = (Re, -Im) of C_t[n] e^{mu lam_t}
        // (the staged C tile); two partial sums (even and odd state tiles)
        // shorten the fp32 chains
        f32x4 ys[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            ys[tt][0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            ys[tt][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kt = 0; kt < NTK; ++kt) {
                if (kt * 16 >= K) break;
                const float4 ch = *reinterpret_cast<const float4 *>(&C_[(tt * 16 + c16) * CP + kt * 16 + 4 * q]);
                f32x4 &a = ys[tt][kt & 1];
                a = mfma4(ch.x, S[kt][0], a);
                a = mfma4(ch.y, S[kt][1], a);
                a = mfma4(ch.z, S[kt][2], a);
                a = mfma4(ch.w, S[kt][3], a);
            }
        }

        // D4: acc[tt] = sum_{s-tile <= tt} M X
        f32x4 acc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int tau = 0; tau < 3; ++tau) {
            const int sT = tau == 2 ? 1 : 0, tT = tau == 0 ? 0 : 1;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[tT] = mfma4(mv[tau][m], X_[(sT * 16 + 4 * q + m) * XP + p0 + c16], acc[tT]);
        }

        // skip term and store: lane (column p0 + c16, rows t = tt*16 + q*4 + v)
        float yv[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                yv[tt][v] = fmaf(Dh, X_[(tt * 16 + 4 * q + v) * XP + p0 + c16],
                                 (ys[tt][0][v] + ys[tt][1][v]) + acc[tt][v]);
        // raw buffer stores whose record count ends at the chunk's last valid step: the
        // hardware drops a ragged tail's stores, so every chunk issues the same 8 stores with
        // no branch around them, and the compiler can count them when it waits for loads
        // issued before them (loads and stores share one counter)
        {
            const int64_t nv = min((int64_t)kT, te - t0);
            const int rec = (int)((nv - 1) * rowX * 4 + 64);   // lane columns < 16: 64 bytes of the last row
            const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(Yg + t0 * rowX, 0, rec, kBufWord3);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv[tt][v]), yr,
                                                          (int)(ylane + (uint32_t)((tt * 16 + v) * rowX) * 4u), 0, 0);
        }

        // D2 + D3
        decay_state<NTK>(S, E, K);
        state_add<NTK, CP, XP>(S, B_, X_, p0, K, lane);

        // stage chunk j+1, start loading chunk j+2
        if (j + 1 < nchunks) {
            st.store(Bs[buf ^ 1], Cs[buf ^ 1], Xs[buf ^ 1], csign);
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

// Workspace: segment states and decays (when there are segments), then the
// chunk records and the M tiles of every (batch, head, chunk).
struct WsLayout {
    Plan pl;
    int64_t nck;
    size_t state, decay, rec, mtile, total;
};
WsLayout ws_layout(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t Nc) {
    WsLayout w{};
    w.pl = plan(batch, L, H, P);
    w.nck = (L + kT - 1) / kT;
    size_t off = 0;
    if (w.pl.nseg > 1) {
        w.state = off;
        off = align256(off + (size_t)(batch * H * w.pl.nseg * P * Nc * 2) * sizeof(float));
        w.decay = off;
        off = align256(off + (size_t)(batch * H * w.pl.nseg * 2) * sizeof(float));
    }
    w.rec = off;
    off = align256(off + (size_t)(batch * H * w.nck) * sizeof(CRec));
    w.mtile = off;
    off += (size_t)(batch * H * w.nck) * 192 * sizeof(f32x4);
    w.total = off;
    return w;
}

template <int KC, bool EXACT, int NW>
void launch_all(const CssdKp &p, hipStream_t stream) {
    const int64_t np = p.batch * p.nck * p.G * ((p.H / p.G + 7) / 8);
    hipLaunchKernelGGL((cssd_prep_kernel<KC, EXACT>), dim3((unsigned)np), dim3(256), 0, stream, p);
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
    return ws_layout(batch, L, nheads, headdim, n_complex).total;
}

int64_t cssd_prep_blocks(int64_t batch, int64_t L, int64_t nheads, int64_t ngroups) {
    return batch * ((L + kT - 1) / kT) * ngroups * ((nheads / ngroups + 7) / 8);
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
    const WsLayout w = ws_layout(p.batch, p.L, p.H, p.P, p.Nc);
    p.nseg = w.pl.nseg;
    p.Ls = w.pl.Ls;
    p.nck = w.nck;
    char *ws = static_cast<char *>(a.workspace);
    if (p.nseg > 1) {
        p.ws_state = reinterpret_cast<float *>(ws + w.state);
        p.ws_decay = reinterpret_cast<float *>(ws + w.decay);
    }
    p.rec = reinterpret_cast<CRec *>(ws + w.rec);
    p.mtile = reinterpret_cast<f32x4 *>(ws + w.mtile);
    if (p.P == 32) launch_k<2>(p, stream);
    else if (p.P == 64) launch_k<4>(p, stream);
    else launch_k<8>(p, stream);
    return hipGetLastError();
}

}  // namespace ssm
