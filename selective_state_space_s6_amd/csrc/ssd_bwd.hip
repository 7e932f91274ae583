// ssd_bwd.hip -- backward pass of the Mamba-2 SSD scan, gfx950.
//
// Gradients of a loss through the scalar-A-per-head recurrence of
// builderforce-memory-engine ssd.js (header comment, ssd_chunk_forward; the
// same package pairs it with a per-chunk backward, ssd_chunk_backward), given
// dy = dL/dy and optionally dh_final = dL/dS_{L-1}.  With G_t = dL/dS_t
// (P x N per (batch, head)):
//   G_t = e^{a_{t+1}} G_{t+1} + dy_t (x) C_t          (G after the last step: dh_final)
//   dx_t  = D dy_t + sigma_t G_t B_t                  dB_t = sigma_t x_t G_t   (summed over
//   dC_t  = dy_t S_t                                  the heads of the group)
//   dh0   = e^{a_0} G_0
// The decay and input-scale gradients come from per-step scalars: with
// cs_t = sum_{k<=t} a_k,
//   dL/dcs_t = dy_t . y_t - x_t . dx_t  (+ <dh_final, h_final> at t = L-1)
//            = C_t . (dy_t S_t) - sigma_t x_t . (G_t B_t)   (the D terms cancel exactly)
//            = C_t . (dy_t S'_t) - sigma_t x_t . (G'_t B_t) with the states less the step's own
//              term, S'_t = S_t - sigma_t x_t B_t^T and G'_t = G_t - dy_t C_t^T: their shares,
//              sigma_t (dy_t.x_t)(C_t.B_t) in both, cancel exactly, so they are left out of both
//              contractions rather than cancelled in rounding (large where a step's decay all
//              but erases the state), and
//   da_t = sum_{t' >= t} dL/dcs_t',   dsigma_t = x_t . (G_t B_t)
//   ddelta_t = da_t A + dsigma_t dsigma/ddelta,  dA = sum da_t delta_t + dsigma_t dsigma/dA.
//
// The sequence of every (batch, head) is cut into segments as in the forward.
// Three walk kernels run over a segment's 32-step chunks with a state in fp32
// MFMA accumulators (v_mfma_f32_16x16x4_f32; every product is exact in fp32):
//   ssdb_walk_f   forward, state S[p][n] (a wave owns 32 columns n):
//                 dC_t = e^{cs_t} dy_t S_in + ((dY X^T) o L) B, the head's share
//   ssdb_walk_r1  backward, state G[p][n] (a wave owns 32 columns n):
//                 dB_t = sigma_t (e^{cs_end-cs_t} x_t G_in + ((X dY^T) o E) C)
//   ssdb_walk_r2  backward, state G^T[n][p] (a wave owns 16 columns p):
//                 u_t = e^{cs_end-cs_t} B_t G_in^T + ((B C^T) o E) dY;  dx = sigma u + D dy
// with L[t,s] = e^{cs_t-cs_s} sigma_s (s <= t) and E[t,t'] = e^{cs_t'-cs_t} (t' >= t).
// In each the accumulator's row index is the contraction index of the
// product that reads it, so it feeds the matrix core without a transpose.
// State-only variants of walk_f and walk_r1 give the segments' own states;
// ssdb_pass_f / ssdb_pass_r turn them into the states entering each segment
// from the left (S) and from the right (G), and ssdb_bnd dots them into the
// exact dL/da at every segment boundary.  ssdb_reduce_heads adds the heads'
// dB, dC shares per group; ssdb_scal runs the reverse sum of dL/dcs over each
// segment from the next boundary's exact value (segments are at most 512 steps,
// which bounds the rounding that sum gathers) and the chain rule for dt,
// A_log, D, dt_bias; ssdb_final adds those over batch and segments.  Every sum
// runs in a fixed order.
#include "device_common.hpp"
#include "launchers.hpp"
#include <algorithm>
#include <type_traits>

namespace ssm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 32;              // steps per chunk
constexpr int kTargetWaves = 3072;  // resident waves wanted (3 per SIMD)
constexpr int kMinSeg = 256;        // shortest segment worth a state round trip
constexpr int kMaxSeg = 512;        // longest segment: bounds the reverse sum behind each ddt

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16x16x32 bf16 MFMA: lane (q = lane/16, i = lane%16) gives row i of A and column i of B at
// K slots 8q..8q+7; the result tile is the 16x16x4 one's (rows 4q..4q+3 of column i)
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}
// two fp32 -> two bf16 (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
// x = hi + mid + lo in bf16, to about 2^-26 of x (each part rounds the remainder of the last)
__device__ __forceinline__ void split3_bf16(const float (&x)[8], u32x4 &hi, u32x4 &mid, u32x4 &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h = pack2_bf16(x[2 * i], x[2 * i + 1]);
        const float r0 = x[2 * i] - __uint_as_float(h << 16), r1 = x[2 * i + 1] - __uint_as_float(h & 0xffff0000u);
        const uint32_t m = pack2_bf16(r0, r1);
        hi[i] = h;
        mid[i] = m;
        lo[i] = pack2_bf16(r0 - __uint_as_float(m << 16), r1 - __uint_as_float(m & 0xffff0000u));
    }
}
// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives the
// four rows sb..sb+3 of column cb + i of a row-major [row][column] bf16 tile
__device__ __forceinline__ uint2 tr_read16(const uint16_t *tile, int pitch, int sb, int cb, int lane) {
    const int i = lane & 15;
    const uint16_t *a = tile + (sb + (i >> 2)) * pitch + cb + 4 * (i & 3);
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4 *)(a)));
}

struct SbKp {
    const uint16_t *x; const float *dt; const float *dt_bias; const float *A_log;
    const uint16_t *B; const uint16_t *C; const float *D; const float *h0;
    const float *dy; const float *dhf;
    float *dx, *ddt, *dB, *dC, *dA_log, *dD, *ddt_bias, *dh0;
    float *Sseg, *Gseg, *dec;          // (batch, H, nseg, P, N) x2, (batch, H, nseg)
    float *dBh, *dCh;                  // (batch, L, H, N): each head's share
    float *dyy, *dsig, *dyx;           // (batch, L, H): C.(dy S'), x.(G' B), dy.x
    float *hfdot;                      // (batch, H)
    double *bnd;                       // (batch, H, nseg): exact dL/da at each segment's first step
    float *pA, *pD, *pT;               // (batch, nseg, H) partial sums
    int64_t batch, L, H, P, N, G, Ls, nseg;
    int mode;                          // 0 ZOH, 1 DT, 2 ONE
    // Mamba-3 trapezoidal form (when trap is set): dt is the step as given,
    // a_t = dt_t aval_t, sigma_t = trap_t dt_t + dt_{t+1} (1 - trap_{t+1}) (the
    // shifted state's input scale), and ssdb_scal leaves dL/da_t in dyy.  The
    // walks also apply the diagonal's correction (its scale is gamma_t, not
    // sigma_t).
    const float *aval, *trap;
    float *dgam;                       // (batch, L, H): (B_t.C_t)(dy_t.x_t), walk R2's diagonal
};

__device__ __forceinline__ float bf(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// per-chunk scalars in LDS
struct Scal {
    float cs[kQ];     // inclusive cumulative sum of a from the chunk start (summed in
    float csl[kQ];    // double, kept as cs + csl): a mask entry's exponent is the difference
                      // of two of them, accurate also where strong decays make the sums large
    float sig[kQ];    // input scale
    float ecs[kQ];    // e^{cs_t}
    float eme[kQ];    // e^{cs_end - cs_t}
    float cd[kQ];     // trapezoidal form: gamma_t - sigma_t (times dy_t.x_t where asked for), else 0
    float csend;
};

// fp64 DPP move: both 32-bit halves moved with the same control (zero where the
// source lane is out of the row or the row is masked off)
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xf, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xf, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// inclusive prefix sum over each 32-lane half, in fp64: row_shr 1, 2, 4, 8 within
// 16-lane rows, then row_bcast:15 into rows 1 and 3
__device__ __forceinline__ double scan32_f64(double v) {
    v += dpp_f64<0x111>(v);
    v += dpp_f64<0x112>(v);
    v += dpp_f64<0x114>(v);
    v += dpp_f64<0x118>(v);
    v += dpp_f64<0x142, 0xa>(v);
    return v;
}
__device__ __forceinline__ double readlane31_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 31);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 31);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// One wave: lanes 0..31 hold steps t0..t0+31 (steps at or past te carry a = 0, sigma = 0).
// with_dyx: the trapezoidal coefficient is multiplied by dy_t.x_t (written by walk R2).
__device__ __forceinline__ void chunk_scalars(Scal &sc, const SbKp &p, int64_t b, int64_t h,
                                              int64_t t0, int64_t te, float bias, float A, int lane,
                                              bool with_dyx = false) {
    const int64_t t = t0 + (lane & 31);
    float a = 0.0f, sg = 0.0f, cd = 0.0f;
    if (lane < kQ && t < te) {
        const int64_t o = (b * p.L + t) * p.H + h;
        if (p.trap) {
            const float dlt = p.dt[o];
            a = dlt * p.aval[o];
            sg = p.trap[o] * dlt;
            if (t + 1 < p.L) {
                const float dn = p.dt[o + p.H], un = 1.0f - p.trap[o + p.H];
                sg = fmaf(dn, un, sg);
                cd = -(dn * un);
            }
            if (with_dyx) cd *= p.dyx[o];
        } else {
            const float dl = softplus(p.dt[o] + bias);
            a = dl * A;
            sg = p.mode == 1 ? dl : (p.mode == 0 ? (a == 0.0f ? dl : dl * (expm1f(a) / a)) : 1.0f);
        }
    }
    const double v = scan32_f64(a);
    const double cend = readlane31_f64(v);
    if (lane < kQ) {
        const float hi = (float)v;
        sc.cs[lane] = hi;
        sc.csl[lane] = (float)(v - (double)hi);
        sc.sig[lane] = sg;
        sc.cd[lane] = cd;
        sc.ecs[lane] = __expf((float)v);
        sc.eme[lane] = __expf((float)(cend - v));
    }
    if (lane == 0) sc.csend = (float)cend;
}

// Sum over the 16 lanes of each DPP row; the total lands in lane 15 of the row.
__device__ __forceinline__ float row_total16(float v) {
    v += dpp_f<0x111>(v);
    v += dpp_f<0x112>(v);
    v += dpp_f<0x114>(v);
    v += dpp_f<0x118>(v);
    return v;
}

// stage rows t0..t0+31 of a (batch, L, R, COLS) tensor slice (row index rr) into LDS as fp32;
// rows at or past te are zero.  COLS is a multiple of 4.
// A lane's 32-bit byte offset, re-read where it is used: the empty asm keeps its
// zero extension next to the access, so that uniform base + offset is the global
// instructions' SGPR-base form rather than a 64-bit VALU add per access
__device__ __forceinline__ uint32_t lane_off(uint32_t o) {
    asm volatile("" : "+v"(o));
    return o;
}

// Stage kQ steps (t0 .. t0+kQ-1, rows past te zero) of one (b, rr) slice of a
// (batch, L, R, COLS) tensor into an fp32 LDS tile: the chunk's first row is a
// uniform base, each lane adds a 32-bit byte offset; bf16 in 16-byte pieces
template <int COLS, int PITCH>
__device__ __forceinline__ void stage_bf16(float (*dst)[PITCH], const uint16_t *src, int64_t b, int64_t L,
                                           int64_t R, int64_t rr, int64_t t0, int64_t te, int tid, int nthr) {
    constexpr int Q8 = COLS / 8;
    const char *row0 = reinterpret_cast<const char *>(src + ((b * L + t0) * R + rr) * COLS);
    const uint32_t rs = (uint32_t)(R * COLS) * 2u;                    // row stride in bytes
    const int nv = (int)min<int64_t>(kQ, te - t0);                     // rows in the sequence
    for (int i = tid; i < kQ * Q8; i += nthr) {
        const int tr = i / Q8, c8 = (i % Q8) * 8;
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (tr < nv) w = *reinterpret_cast<const uint4 *>(row0 + lane_off((uint32_t)tr * rs + (uint32_t)c8 * 2u));
        *reinterpret_cast<float4 *>(&dst[tr][c8]) =
            make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                        __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
        *reinterpret_cast<float4 *>(&dst[tr][c8 + 4]) =
            make_float4(__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xffff0000u),
                        __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xffff0000u));
    }
}
template <int COLS, int PITCH>
__device__ __forceinline__ void stage_f32(float (*dst)[PITCH], const float *src, int64_t b, int64_t L,
                                          int64_t R, int64_t rr, int64_t t0, int64_t te, int tid, int nthr) {
    constexpr int Q4 = COLS / 4;
    const char *row0 = reinterpret_cast<const char *>(src + ((b * L + t0) * R + rr) * COLS);
    const uint32_t rs = (uint32_t)(R * COLS) * 4u;
    const int nv = (int)min<int64_t>(kQ, te - t0);
    for (int i = tid; i < kQ * Q4; i += nthr) {
        const int tr = i / Q4, c4 = (i % Q4) * 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tr < nv) v = *reinterpret_cast<const float4 *>(row0 + lane_off((uint32_t)tr * rs + (uint32_t)c4 * 4u));
        *reinterpret_cast<float4 *>(&dst[tr][c4]) = v;
    }
}

// The same chunk rows of a bf16 tensor kept as bf16 in LDS (16-byte pieces)
template <int COLS, int PITCH>
__device__ __forceinline__ void stage_bf16_raw(uint16_t (*dst)[PITCH], const uint16_t *src, int64_t b, int64_t L,
                                               int64_t R, int64_t rr, int64_t t0, int64_t te, int tid, int nthr) {
    constexpr int Q8 = COLS / 8;
    const char *row0 = reinterpret_cast<const char *>(src + ((b * L + t0) * R + rr) * COLS);
    const uint32_t rs = (uint32_t)(R * COLS) * 2u;
    const int nv = (int)min<int64_t>(kQ, te - t0);
    for (int i = tid; i < kQ * Q8; i += nthr) {
        const int tr = i / Q8, c8 = (i % Q8) * 8;
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (tr < nv) w = *reinterpret_cast<const uint4 *>(row0 + lane_off((uint32_t)tr * rs + (uint32_t)c8 * 2u));
        *reinterpret_cast<uint4 *>(&dst[tr][c8]) = w;
    }
}

// Element (row 16 ti + 4 r + v, column) of a chunk tile in global memory: the
// uniform chunk base plus rows (16 ti + v) whole rows (SGPRs), and the lane's
// rows 4 r and its column as a 32-bit byte offset
template <typename T>
__device__ __forceinline__ T &chunk_elem(T *base0, uint32_t row_bytes, int urows, uint32_t lane_bytes) {
    using B = std::conditional_t<std::is_const_v<T>, const char, char>;
    return *reinterpret_cast<T *>(reinterpret_cast<B *>(base0) + (uint64_t)urows * row_bytes + lane_off(lane_bytes));
}

__device__ __forceinline__ int64_t seg_off(const SbKp &p, int64_t b, int64_t h, int64_t k) {
    return ((b * p.H + h) * p.nseg + k) * p.P * p.N;
}

// ------------------------------------------------------------------ walk F
// STATE: segments 0..nseg-2 from a zero state, writing their own final states
// and decays.  Otherwise: every segment from its entering state, writing the
// head's dC share, the per-step scalar C_t . dC_t, and <dh_final, h_final>.
template <int P, int N, bool STATE>
__global__ void __launch_bounds__(64 * (N / 32))
ssdb_walk_f(SbKp p) {
    constexpr int NW = N / 32, PT = P / 16, NTH = 64 * NW;
    __shared__ __attribute__((aligned(16))) float sX[kQ][P + 4];
    __shared__ __attribute__((aligned(16))) float sY[STATE ? 1 : kQ][P + 4];
    __shared__ __attribute__((aligned(16))) float sB[kQ][N + 4];
    __shared__ __attribute__((aligned(16))) float sM[STATE ? 1 : kQ][kQ + 4];
    __shared__ float sRed[NW][kQ];
    __shared__ float sDg[STATE ? 1 : kQ];   // the own term's coefficient, sigma_t (dy_t.x_t)
    __shared__ Scal sc;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane >> 4, c16 = lane & 15;
    const int64_t nsl = STATE ? p.nseg - 1 : p.nseg;
    const int64_t k = blockIdx.x % nsl, bh = blockIdx.x / nsl;
    const int64_t b = bh / p.H, h = bh % p.H, g = h * p.G / p.H;
    const int64_t T0 = k * p.Ls, T1 = min(T0 + p.Ls, p.L);
    const float A = p.A_log ? -expf(p.A_log[h]) : 0.0f;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;

    // S tile (pt, nt): rows p = 16 pt + 4 r + v, column n = 32 w + 16 nt + c16
    f32x4 S[PT][2];
    {
        const float *src = nullptr;
        if constexpr (!STATE) src = k == 0 ? p.h0 + (p.h0 ? (b * p.H + h) * P * N : 0) : p.Sseg + seg_off(p, b, h, k);
        if (k == 0 && !p.h0) src = nullptr;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    S[pt][nt][v] = src ? src[(16 * pt + 4 * r + v) * N + 32 * w + 16 * nt + c16] : 0.0f;
    }
    float sumA = 0.0f;
    for (int64_t t0 = T0; t0 < T1; t0 += kQ) {
        stage_bf16<P, P + 4>(sX, p.x, b, p.L, p.H, h, t0, T1, tid, NTH);
        stage_bf16<N, N + 4>(sB, p.B, b, p.L, p.G, g, t0, T1, tid, NTH);
        if constexpr (!STATE) stage_f32<P, P + 4>(sY, p.dy, b, p.L, p.H, h, t0, T1, tid, NTH);
        if (w == 0) chunk_scalars(sc, p, b, h, t0, T1, bias, A, lane, !STATE);
        __syncthreads();
        const float csend = sc.csend;
        if constexpr (!STATE) {
            // (dY X^T) o L, lower-triangular tiles (0,0), (1,0), (1,1) of [t][s]
            for (int tau = w; tau < 3; tau += NW) {
                const int ti = tau == 0 ? 0 : 1, si = tau == 2 ? 1 : 0;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const float4 a4 = *reinterpret_cast<const float4 *>(&sY[16 * ti + c16][16 * pt + 4 * r]);
                    const float4 b4 = *reinterpret_cast<const float4 *>(&sX[16 * si + c16][16 * pt + 4 * r]);
                    acc = mfma4(a4.x, b4.x, acc);
                    acc = mfma4(a4.y, b4.y, acc);
                    acc = mfma4(a4.z, b4.z, acc);
                    acc = mfma4(a4.w, b4.w, acc);
                }
                const int s = 16 * si + c16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t = 16 * ti + 4 * r + v;
                    const float m = s <= t ? acc[v] * __expf((sc.cs[t] - sc.cs[s]) + (sc.csl[t] - sc.csl[s])) * sc.sig[s] : 0.0f;
                    if (s == t) sDg[t] = p.trap ? m + sc.cd[t] : m;   // with the trapezoidal diagonal's share
                    sM[t][s] = s == t ? 0.0f : m;     // the step's own term enters dC below
                }
            }
            __syncthreads();
            // dC tiles (ti, nt): state part scaled by e^{cs_t}, then the intra-chunk part
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const float4 a4 = *reinterpret_cast<const float4 *>(&sY[16 * ti + c16][16 * pt + 4 * r]);
                        acc = mfma4(a4.x, S[pt][nt][0], acc);
                        acc = mfma4(a4.y, S[pt][nt][1], acc);
                        acc = mfma4(a4.z, S[pt][nt][2], acc);
                        acc = mfma4(a4.w, S[pt][nt][3], acc);
                    }
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] *= sc.ecs[16 * ti + 4 * r + v];
                    const int n = 32 * w + 16 * nt + c16;
#pragma unroll
                    for (int si = 0; si <= ti; ++si) {
                        const float4 a4 = *reinterpret_cast<const float4 *>(&sM[16 * ti + c16][16 * si + 4 * r]);
                        acc = mfma4(a4.x, sB[16 * si + 4 * r + 0][n], acc);
                        acc = mfma4(a4.y, sB[16 * si + 4 * r + 1][n], acc);
                        acc = mfma4(a4.z, sB[16 * si + 4 * r + 2][n], acc);
                        acc = mfma4(a4.w, sB[16 * si + 4 * r + 3][n], acc);
                    }
                    float *dC0 = p.dCh + ((b * p.L + t0) * p.H + h) * N;
                    const uint16_t *C0 = p.C + ((b * p.L + t0) * p.G + g) * N;
                    const uint32_t rsD = (uint32_t)(p.H * N) * 4u, rsC = (uint32_t)(p.G * N) * 2u;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int tl = 16 * ti + 4 * r + v;
                        const int64_t t = t0 + tl;
                        if (t < T1) {
                            // acc is dy_t S'_t (the state less the step's own term), whose C_t dot
                            // product is the step's scalar; dC_t adds the own term, sigma_t
                            // (dy_t.x_t) B_t, and in the trapezoidal form the diagonal's share
                            // (gamma_t - sigma_t)(dy_t.x_t) k_t
                            chunk_elem(dC0, rsD, 16 * ti + v, (uint32_t)(4 * r) * rsD + (uint32_t)n * 4u) =
                                fmaf(sDg[tl], sB[tl][n], acc[v]);
                            part[v] += bf(chunk_elem(C0, rsC, 16 * ti + v, (uint32_t)(4 * r) * rsC + (uint32_t)n * 2u)) *
                                       acc[v];
                        }
                    }
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float tot = row_total16(part[v]);
                    if (c16 == 15) sRed[w][16 * ti + 4 * r + v] = tot;
                }
            }
        }
        // S <- e^{cs_end} S + X^T (w o B), w_s = e^{cs_end - cs_s} sigma_s
        const float eend = __expf(csend);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) S[pt][nt] *= eend;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int s = 16 * st + 4 * r + v;
                const float ws = sc.eme[s] * sc.sig[s];
                const float b0 = sB[s][32 * w + c16] * ws, b1 = sB[s][32 * w + 16 + c16] * ws;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const float a = sX[s][16 * pt + c16];
                    S[pt][0] = mfma4(a, b0, S[pt][0]);
                    S[pt][1] = mfma4(a, b1, S[pt][1]);
                }
            }
        sumA += csend;
        __syncthreads();
        if constexpr (!STATE) {
            if (tid < kQ && t0 + tid < T1) {
                float s = 0.0f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) s += sRed[ww][tid];
                p.dyy[(b * p.L + t0 + tid) * p.H + h] = s;
            }
        }
    }
    if constexpr (STATE) {
        float *dst = p.Sseg + seg_off(p, b, h, k);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) dst[(16 * pt + 4 * r + v) * N + 32 * w + 16 * nt + c16] = S[pt][nt][v];
        if (tid == 0) p.dec[(b * p.H + h) * p.nseg + k] = expf(sumA);
    } else {
        if (k == p.nseg - 1) {
            // <dh_final, h_final>
            float part = 0.0f;
            if (p.dhf) {
                const float *src = p.dhf + (b * p.H + h) * P * N;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            part += src[(16 * pt + 4 * r + v) * N + 32 * w + 16 * nt + c16] * S[pt][nt][v];
            }
            // wave total (lanes in a fixed order), then over waves; sRed may still
            // be read for the last chunk's per-step sums until every wave is here
            part = row_total16(part);
            __syncthreads();
            if (c16 == 15) sRed[w][r] = part;
            __syncthreads();
            if (tid == 0) {
                float s = 0.0f;
                for (int ww = 0; ww < NW; ++ww)
                    for (int rr = 0; rr < 4; ++rr) s += sRed[ww][rr];
                p.hfdot[b * p.H + h] = s;
            }
        }
    }
}

// ----------------------------------------------------------------- walk R1
// STATE: segments 1..nseg-1 backward from a zero gradient, writing their own
// gradient states (and the last segment's decay).  Otherwise: every segment
// backward from the gradient entering from the right, writing the head's dB
// share and, at the start of the sequence, dh0.
// The bf16 state update's operands take the walk a few VGPRs past 128 unless 4 waves per
// SIMD are asked for, which the compiler then meets without spilling.
template <int P, int N, bool STATE>
__global__ void __launch_bounds__(64 * (N / 32)) __attribute__((amdgpu_waves_per_eu(P <= 64 && !STATE ? 4 : 1)))
ssdb_walk_r1(SbKp p) {
    constexpr int NW = N / 32, PT = P / 16, NTH = 64 * NW;
    __shared__ __attribute__((aligned(16))) float sX[STATE ? 1 : kQ][P + 4];
    __shared__ __attribute__((aligned(16))) float sY[kQ][P + 4];
    __shared__ __attribute__((aligned(16))) uint16_t sC[kQ][N + 8];   // bf16, exact
    __shared__ __attribute__((aligned(16))) float sM[STATE ? 1 : kQ][kQ + 4];
    __shared__ Scal sc;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane >> 4, c16 = lane & 15;
    const int64_t nsl = STATE ? p.nseg - 1 : p.nseg;
    const int64_t k = (STATE ? 1 : 0) + blockIdx.x % nsl, bh = blockIdx.x / nsl;
    const int64_t b = bh / p.H, h = bh % p.H, g = h * p.G / p.H;
    const int64_t T0 = k * p.Ls, T1 = min(T0 + p.Ls, p.L);
    const float A = p.A_log ? -expf(p.A_log[h]) : 0.0f;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;

    // G tile (pt, nt): rows p = 16 pt + 4 r + v, column n = 32 w + 16 nt + c16
    f32x4 Gs[PT][2];
    {
        const float *src = nullptr;
        if constexpr (!STATE) {
            if (k == p.nseg - 1) src = p.dhf ? p.dhf + (b * p.H + h) * P * N : nullptr;
            else src = p.Gseg + seg_off(p, b, h, k);
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    Gs[pt][nt][v] = src ? src[(16 * pt + 4 * r + v) * N + 32 * w + 16 * nt + c16] : 0.0f;
    }
    float sumA = 0.0f;
    const int64_t nch = (T1 - T0 + kQ - 1) / kQ;
    for (int64_t ci = nch - 1; ci >= 0; --ci) {
        const int64_t t0 = T0 + ci * kQ;
        stage_f32<P, P + 4>(sY, p.dy, b, p.L, p.H, h, t0, T1, tid, NTH);
        stage_bf16_raw<N, N + 8>(sC, p.C, b, p.L, p.G, g, t0, T1, tid, NTH);
        if constexpr (!STATE) stage_bf16<P, P + 4>(sX, p.x, b, p.L, p.H, h, t0, T1, tid, NTH);
        if (w == 0) chunk_scalars(sc, p, b, h, t0, T1, bias, A, lane, !STATE);
        __syncthreads();
        const float csend = sc.csend;
        if constexpr (!STATE) {
            // (X dY^T) o E, upper-triangular tiles (0,0), (0,1), (1,1) of [t][t']
            for (int tau = w; tau < 3; tau += NW) {
                const int ti = tau == 2 ? 1 : 0, tj = tau == 0 ? 0 : 1;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const float4 a4 = *reinterpret_cast<const float4 *>(&sX[16 * ti + c16][16 * pt + 4 * r]);
                    const float4 b4 = *reinterpret_cast<const float4 *>(&sY[16 * tj + c16][16 * pt + 4 * r]);
                    acc = mfma4(a4.x, b4.x, acc);
                    acc = mfma4(a4.y, b4.y, acc);
                    acc = mfma4(a4.z, b4.z, acc);
                    acc = mfma4(a4.w, b4.w, acc);
                }
                const int tp = 16 * tj + c16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t = 16 * ti + 4 * r + v;
                    sM[t][tp] = tp >= t ? acc[v] * __expf((sc.cs[tp] - sc.cs[t]) + (sc.csl[tp] - sc.csl[t])) : 0.0f;
                }
            }
            __syncthreads();
            // dB tiles (ti, nt)
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const float4 a4 = *reinterpret_cast<const float4 *>(&sX[16 * ti + c16][16 * pt + 4 * r]);
                        acc = mfma4(a4.x, Gs[pt][nt][0], acc);
                        acc = mfma4(a4.y, Gs[pt][nt][1], acc);
                        acc = mfma4(a4.z, Gs[pt][nt][2], acc);
                        acc = mfma4(a4.w, Gs[pt][nt][3], acc);
                    }
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] *= sc.eme[16 * ti + 4 * r + v];
                    const int n = 32 * w + 16 * nt + c16;
#pragma unroll
                    for (int tj = ti; tj < 2; ++tj) {
                        const float4 a4 = *reinterpret_cast<const float4 *>(&sM[16 * ti + c16][16 * tj + 4 * r]);
                        acc = mfma4(a4.x, bf(sC[16 * tj + 4 * r + 0][n]), acc);
                        acc = mfma4(a4.y, bf(sC[16 * tj + 4 * r + 1][n]), acc);
                        acc = mfma4(a4.z, bf(sC[16 * tj + 4 * r + 2][n]), acc);
                        acc = mfma4(a4.w, bf(sC[16 * tj + 4 * r + 3][n]), acc);
                    }
                    float *dB0 = p.dBh + ((b * p.L + t0) * p.H + h) * N;
                    const uint32_t rsD = (uint32_t)(p.H * N) * 4u;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int tl = 16 * ti + 4 * r + v;
                        const int64_t t = t0 + tl;
                        if (t < T1) {
                            // plus the trapezoidal diagonal's dk_t += (gamma_t - sigma_t)(dy_t.x_t) q_t
                            const float db = acc[v] * sc.sig[tl];
                            chunk_elem(dB0, rsD, 16 * ti + v, (uint32_t)(4 * r) * rsD + (uint32_t)n * 4u) =
                                p.trap ? fmaf(sc.cd[tl], bf(sC[tl][n]), db) : db;
                        }
                    }
                }
        }
        // G <- e^{cs_end} G + (e^{cs} o dY)^T C on bf16 MFMA: C read transposed from the bf16
        // tile, e^{cs} o dY split into three bf16 terms (fp32-exact), the chunk's 32 steps in
        // K order (4r..4r+3, 16+4r..16+4r+3) on both operands
        const float eend = __expf(csend);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) Gs[pt][nt] *= eend;
        {
            u32x4 Cf[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const uint2 a0 = tr_read16(&sC[0][0], N + 8, 4 * r, 32 * w + 16 * nt, lane);
                const uint2 a1 = tr_read16(&sC[0][0], N + 8, 16 + 4 * r, 32 * w + 16 * nt, lane);
                Cf[nt] = u32x4{a0.x, a0.y, a1.x, a1.y};
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                float av[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int s = (i < 4 ? 0 : 16) + 4 * r + (i & 3);
                    av[i] = sY[s][16 * pt + c16] * sc.ecs[s];
                }
                u32x4 Ah, Am, Al;
                split3_bf16(av, Ah, Am, Al);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    Gs[pt][nt] = mfma_bf16(Ah, Cf[nt], Gs[pt][nt]);
                    Gs[pt][nt] = mfma_bf16(Am, Cf[nt], Gs[pt][nt]);
                    Gs[pt][nt] = mfma_bf16(Al, Cf[nt], Gs[pt][nt]);
                }
            }
        }
        sumA += csend;
        __syncthreads();
    }
    if constexpr (STATE) {
        float *dst = p.Gseg + seg_off(p, b, h, k);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) dst[(16 * pt + 4 * r + v) * N + 32 * w + 16 * nt + c16] = Gs[pt][nt][v];
        if (tid == 0 && k == p.nseg - 1) p.dec[(b * p.H + h) * p.nseg + k] = expf(sumA);
    } else if (k == 0 && p.dh0) {
        float *dst = p.dh0 + (b * p.H + h) * P * N;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) dst[(16 * pt + 4 * r + v) * N + 32 * w + 16 * nt + c16] = Gs[pt][nt][v];
    }
}

// ----------------------------------------------------------------- walk R2
// Every segment backward from the gradient entering from the right, with the
// gradient held transposed (G^T[n][p]; a wave owns 16 columns p): writes dx
// and the per-step scalars x . u and dy . x.
template <int P, int N>
__global__ void __launch_bounds__(64 * (P / 16))
ssdb_walk_r2(SbKp p) {
    constexpr int NW = P / 16, NT = N / 16, NTH = 64 * NW;
    __shared__ __attribute__((aligned(16))) float sB[kQ][N + 4];
    // C stays bf16 in LDS (it is exact there): the group's LDS then allows 4 groups per CU
    __shared__ __attribute__((aligned(16))) uint16_t sC[kQ][N + 8];
    __shared__ __attribute__((aligned(16))) float sY[kQ][P + 4];
    __shared__ __attribute__((aligned(16))) float sM[kQ][kQ + 4];
    __shared__ float sRed[NW][2][kQ];
    __shared__ float sDg[kQ];   // the mask's diagonal, B_t.C_t
    __shared__ Scal sc;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane >> 4, c16 = lane & 15;
    const int64_t k = blockIdx.x % p.nseg, bh = blockIdx.x / p.nseg;
    const int64_t b = bh / p.H, h = bh % p.H, g = h * p.G / p.H;
    const int64_t T0 = k * p.Ls, T1 = min(T0 + p.Ls, p.L);
    const float A = p.A_log ? -expf(p.A_log[h]) : 0.0f;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const float Dh = p.D ? p.D[h] : 0.0f;
    const int pc = 16 * w + c16;                       // this lane's column p

    // G^T tile nt: rows n = 16 nt + 4 r + v, column p = 16 w + c16
    f32x4 Gt[NT];
    {
        const float *src = k == p.nseg - 1 ? (p.dhf ? p.dhf + (b * p.H + h) * P * N : nullptr)
                                           : p.Gseg + seg_off(p, b, h, k);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) Gt[nt][v] = src ? src[pc * N + 16 * nt + 4 * r + v] : 0.0f;
    }
    const int64_t nch = (T1 - T0 + kQ - 1) / kQ;
    for (int64_t ci = nch - 1; ci >= 0; --ci) {
        const int64_t t0 = T0 + ci * kQ;
        stage_bf16<N, N + 4>(sB, p.B, b, p.L, p.G, g, t0, T1, tid, NTH);
        stage_bf16_raw<N, N + 8>(sC, p.C, b, p.L, p.G, g, t0, T1, tid, NTH);
        stage_f32<P, P + 4>(sY, p.dy, b, p.L, p.H, h, t0, T1, tid, NTH);
        if (w == 0) chunk_scalars(sc, p, b, h, t0, T1, bias, A, lane);
        __syncthreads();
        const float csend = sc.csend;
        // (B C^T) o E, upper-triangular tiles (0,0), (0,1), (1,1) of [t][t']
        for (int tau = w; tau < 3; tau += NW) {
            const int ti = tau == 2 ? 1 : 0, tj = tau == 0 ? 0 : 1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NT; ++kt) {
                const float4 a4 = *reinterpret_cast<const float4 *>(&sB[16 * ti + c16][16 * kt + 4 * r]);
                const uint2 c2 = *reinterpret_cast<const uint2 *>(&sC[16 * tj + c16][16 * kt + 4 * r]);
                const float4 b4 = make_float4(__uint_as_float(c2.x << 16), __uint_as_float(c2.x & 0xffff0000u),
                                              __uint_as_float(c2.y << 16), __uint_as_float(c2.y & 0xffff0000u));
                acc = mfma4(a4.x, b4.x, acc);
                acc = mfma4(a4.y, b4.y, acc);
                acc = mfma4(a4.z, b4.z, acc);
                acc = mfma4(a4.w, b4.w, acc);
            }
            const int tp = 16 * tj + c16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 16 * ti + 4 * r + v;
                const float m = tp >= t ? acc[v] * __expf((sc.cs[tp] - sc.cs[t]) + (sc.csl[tp] - sc.csl[t])) : 0.0f;
                if (tp == t) sDg[t] = m;
                sM[t][tp] = tp == t ? 0.0f : m;   // the step's own term enters dx below
            }
        }
        __syncthreads();
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float4 a4 = *reinterpret_cast<const float4 *>(&sB[16 * ti + c16][16 * nt + 4 * r]);
                acc = mfma4(a4.x, Gt[nt][0], acc);
                acc = mfma4(a4.y, Gt[nt][1], acc);
                acc = mfma4(a4.z, Gt[nt][2], acc);
                acc = mfma4(a4.w, Gt[nt][3], acc);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] *= sc.eme[16 * ti + 4 * r + v];
#pragma unroll
            for (int tj = ti; tj < 2; ++tj) {
                const float4 a4 = *reinterpret_cast<const float4 *>(&sM[16 * ti + c16][16 * tj + 4 * r]);
                acc = mfma4(a4.x, sY[16 * tj + 4 * r + 0][pc], acc);
                acc = mfma4(a4.y, sY[16 * tj + 4 * r + 1][pc], acc);
                acc = mfma4(a4.z, sY[16 * tj + 4 * r + 2][pc], acc);
                acc = mfma4(a4.w, sY[16 * tj + 4 * r + 3][pc], acc);
            }
            // acc = u'_t = G'_t B_t (the gradient state less the step's own term):
            // dx = sigma (u' + (B_t.C_t) dy) + D dy, and the per-step sums over p
            const uint16_t *X0 = p.x + ((b * p.L + t0) * p.H + h) * P;
            float *dX0 = p.dx + ((b * p.L + t0) * p.H + h) * P;
            const uint32_t rsX = (uint32_t)(p.H * P) * 2u, rsDX = (uint32_t)(p.H * P) * 4u;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tl = 16 * ti + 4 * r + v;
                const int64_t t = t0 + tl;
                const float dyv = sY[tl][pc];
                float xv = 0.0f, dxv = 0.0f;
                if (t < T1) {
                    xv = bf(chunk_elem(X0, rsX, 16 * ti + v, (uint32_t)(4 * r) * rsX + (uint32_t)pc * 2u));
                    // trapezoidal diagonal: dx_t += (gamma_t - sigma_t)(q_t.k_t) dy_t, with
                    // q_t.k_t the diagonal of (B C^T) o E (its decay factor there is e^0)
                    const float dg = sDg[tl];
                    const float sk = fmaf(sc.sig[tl], dg, p.trap ? fmaf(sc.cd[tl], dg, Dh) : Dh);
                    dxv = fmaf(sc.sig[tl], acc[v], sk * dyv);
                    chunk_elem(dX0, rsDX, 16 * ti + v, (uint32_t)(4 * r) * rsDX + (uint32_t)pc * 4u) = dxv;
                }
                const float s0 = row_total16(xv * acc[v]);
                const float s2 = row_total16(dyv * xv);
                if (c16 == 15) {
                    sRed[w][0][tl] = s0;
                    sRed[w][1][tl] = s2;
                }
            }
        }
        // G^T <- e^{cs_end} G^T + C^T (e^{cs} o dY) on bf16 MFMA: C^T read transposed from
        // the bf16 C tile, e^{cs} o dY split into three bf16 terms (fp32-exact), the chunk's
        // 32 steps in K order (4r..4r+3, 16+4r..16+4r+3) on both operands
        const float eend = __expf(csend);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) Gt[nt] *= eend;
        {
            float bb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int s = (i < 4 ? 0 : 16) + 4 * r + (i & 3);
                bb[i] = sY[s][pc] * sc.ecs[s];
            }
            u32x4 Bh, Bm, Bl;
            split3_bf16(bb, Bh, Bm, Bl);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const uint2 a0 = tr_read16(&sC[0][0], N + 8, 4 * r, 16 * nt, lane);
                const uint2 a1 = tr_read16(&sC[0][0], N + 8, 16 + 4 * r, 16 * nt, lane);
                const u32x4 Af{a0.x, a0.y, a1.x, a1.y};
                Gt[nt] = mfma_bf16(Af, Bh, Gt[nt]);
                Gt[nt] = mfma_bf16(Af, Bm, Gt[nt]);
                Gt[nt] = mfma_bf16(Af, Bl, Gt[nt]);
            }
        }
        __syncthreads();
        if (tid < kQ && t0 + tid < T1) {
            float s0 = 0.0f, s2 = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) { s0 += sRed[ww][0][tid]; s2 += sRed[ww][1][tid]; }
            const int64_t o = (b * p.L + t0 + tid) * p.H + h;
            p.dsig[o] = s0;
            p.dyx[o] = s2;
            p.dgam[o] = sDg[tid] * s2;
        }
    }
}

// ------------------------------------------------------------------ passes
// S entering each segment: S_in[0] = h0, S_in[k+1] = dec[k] S_in[k] + S_loc[k].
__global__ void __launch_bounds__(256) ssdb_pass_f(SbKp p) {
    const int64_t PN = p.P * p.N, tot = p.batch * p.H * PN;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= tot) return;
    const int64_t bh = i / PN, e = i % PN;
    float s = p.h0 ? p.h0[bh * PN + e] : 0.0f;
    for (int64_t k = 0; k < p.nseg; ++k) {
        float *q = p.Sseg + (bh * p.nseg + k) * PN + e;
        const float loc = k < p.nseg - 1 ? *q : 0.0f;
        *q = s;
        if (k < p.nseg - 1) s = fmaf(p.dec[bh * p.nseg + k], s, loc);
    }
}
// G entering each segment from the right: G_in[nseg-1] = dh_final,
// G_in[k-1] = dec[k] G_in[k] + G_loc[k].
__global__ void __launch_bounds__(256) ssdb_pass_r(SbKp p) {
    const int64_t PN = p.P * p.N, tot = p.batch * p.H * PN;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= tot) return;
    const int64_t bh = i / PN, e = i % PN;
    float gv = p.dhf ? p.dhf[bh * PN + e] : 0.0f;
    for (int64_t k = p.nseg - 1; k >= 0; --k) {
        float *q = p.Gseg + (bh * p.nseg + k) * PN + e;
        const float loc = k >= 1 ? *q : 0.0f;
        *q = gv;
        if (k >= 1) gv = fmaf(p.dec[bh * p.nseg + k], gv, loc);
    }
}

// dB, dC: the heads' shares added per group, heads in order
__global__ void __launch_bounds__(256) ssdb_reduce_heads(SbKp p) {
    const int64_t tot = p.batch * p.L * p.G * p.N;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= tot) return;
    const int64_t n = i % p.N, rest = i / p.N, g = rest % p.G, bt = rest / p.G;
    const int64_t hpg = p.H / p.G;
    float sb = 0.0f, scv = 0.0f;
    for (int64_t j = 0; j < hpg; ++j) {
        const int64_t o = (bt * p.H + g * hpg + j) * p.N + n;
        sb += p.dBh[o];
        scv += p.dCh[o];
    }
    p.dB[i] = sb;
    p.dC[i] = scv;
}

// phi1'(z) for the zero-order hold's dsigma/dA: series below |z| = 1/4
// (truncation < 2e-9 relative), the closed form above.
__device__ __forceinline__ float dphi1f(float z) {
    if (fabsf(z) < 0.25f) {
        float q = fmaf(z, 1.0f / 5760.0f, 1.0f / 840.0f);
        q = fmaf(z, q, 1.0f / 144.0f);
        q = fmaf(z, q, 1.0f / 30.0f);
        q = fmaf(z, q, 1.0f / 8.0f);
        q = fmaf(z, q, 1.0f / 3.0f);
        return fmaf(z, q, 0.5f);
    }
    const float e = __expf(z);
    return fmaf(e, z - 1.0f, 1.0f) / (z * z);
}

// dL/da at the first step T0 of every segment k >= 1, exactly:
// e^{a_T0} <G_T0, S_{T0-1}> = <G entering segment k-1 from the right, S entering segment k>.
// One block per (batch, head, k); a fixed-order tree over the P*N products.
constexpr int kBndThreads = 256;
__global__ void __launch_bounds__(kBndThreads) ssdb_bnd(SbKp p) {
    __shared__ double sR[kBndThreads];
    const int tid = threadIdx.x;
    const int64_t k = 1 + blockIdx.x % (p.nseg - 1), bh = blockIdx.x / (p.nseg - 1);
    const int64_t PN = p.P * p.N;
    const float *gs = p.Gseg + (bh * p.nseg + k - 1) * PN;
    const float *ss = p.Sseg + (bh * p.nseg + k) * PN;
    double acc = 0.0;
    for (int64_t e = tid; e < PN; e += kBndThreads) acc += (double)gs[e] * (double)ss[e];
    sR[tid] = acc;
    __syncthreads();
    for (int st = kBndThreads / 2; st > 0; st >>= 1) {
        if (tid < st) sR[tid] += sR[tid + st];
        __syncthreads();
    }
    if (tid == 0) p.bnd[bh * p.nseg + k] = sR[0];
}

// Per (batch, segment, head), one 64-thread block; thread j owns a contiguous
// run of the segment's steps.  The reverse sum of dL/dcs over the segment,
// started from the exact boundary value of the next segment (0 after the
// last), gives da_t (runs summed in fp64, a fixed-order suffix over the
// threads); then the chain rule to ddt and the segment's partial sums of
// dA_log / A, dD and ddt_bias.
constexpr int kScalThreads = 64;
__global__ void __launch_bounds__(kScalThreads) ssdb_scal(SbKp p) {
    __shared__ double sTot[kScalThreads];
    __shared__ float sR[3][kScalThreads];
    const int tid = threadIdx.x;
    const int64_t i = blockIdx.x;
    const int64_t h = i % p.H, bk = i / p.H, k = bk % p.nseg, b = bk / p.nseg;
    const int64_t bh = b * p.H + h;
    const float A = p.A_log ? -expf(p.A_log[h]) : 0.0f;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const int64_t T0 = k * p.Ls, T1 = min(T0 + p.Ls, p.L);
    const int64_t per = (T1 - T0 + kScalThreads - 1) / kScalThreads;
    const int64_t lo = min(T1, T0 + tid * per), hi = min(T1, lo + per);
    // dL/dcs_t = dy_t.y_t - x_t.dx_t = C_t.dC_t - sigma_t x_t.u_t: the skip term D
    // cancels exactly, so it is left out rather than added and subtracted in fp32
    auto sigma = [&](float dl, float a) __attribute__((always_inline)) {
        return p.mode == 1 ? dl : (p.mode == 0 ? (a == 0.0f ? dl : dl * (expm1f(a) / a)) : 1.0f);
    };
    auto dcs = [&](int64_t t, float sg) __attribute__((always_inline)) {
        const int64_t o = (b * p.L + t) * p.H + h;
        double v = (double)p.dyy[o] - (double)sg * (double)p.dsig[o];
        if (t == p.L - 1) v += (double)p.hfdot[bh];
        return v;
    };
    // trapezoidal form: sigma of step t from its own and the next step's inputs
    auto sigma_trap = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t o = (b * p.L + t) * p.H + h;
        float sg = p.trap[o] * p.dt[o];
        if (t + 1 < p.L) sg = fmaf(p.dt[o + p.H], 1.0f - p.trap[o + p.H], sg);
        return sg;
    };
    double loc = 0.0;
    for (int64_t t = hi - 1; t >= lo; --t) {
        if (p.trap) {
            loc += dcs(t, sigma_trap(t));
        } else {
            const float dl = softplus(p.dt[(b * p.L + t) * p.H + h] + bias);
            loc += dcs(t, sigma(dl, dl * A));
        }
    }
    sTot[tid] = loc;
    __syncthreads();
    double carry = k + 1 < p.nseg ? p.bnd[bh * p.nseg + k + 1] : 0.0;
    for (int j = kScalThreads - 1; j > tid; --j) carry += sTot[j];
    float aA = 0.0f, aD = 0.0f, aT = 0.0f;
    if (p.trap) {     // dL/da_t goes to dyy (read above for this step only); the chain to dt follows
        for (int64_t t = hi - 1; t >= lo; --t) {
            const int64_t o = (b * p.L + t) * p.H + h;
            carry += dcs(t, sigma_trap(t));
            p.dyy[o] = (float)carry;
            aD += p.dyx[o];
        }
    }
    for (int64_t t = p.trap ? lo - 1 : hi - 1; t >= lo; --t) {
        const int64_t o = (b * p.L + t) * p.H + h;
        const float x = p.dt[o] + bias;
        const float dl = softplus(x);
        const float a = dl * A;
        const float sg = sigma(dl, a);
        float dsd, dsa;
        if (p.mode == 1) { dsd = 1.0f; dsa = 0.0f; }
        else if (p.mode == 0) { dsd = __expf(a); dsa = dl * dl * dphi1f(a); }
        else { dsd = 0.0f; dsa = 0.0f; }
        carry += dcs(t, sg);                         // da_t = sum_{t' >= t} dL/dcs_t'
        const float da = (float)carry;
        const float ds = p.dsig[o] + p.dgam[o];          // x_t.(G_t B_t), the own term included
        const float ddl = fmaf(da, A, ds * dsd);
        aA = fmaf(da, dl, fmaf(ds, dsa, aA));
        const float g = ddl * (1.0f / (1.0f + __expf(-x)));
        p.ddt[o] = g;
        aT += g;
        aD += p.dyx[o];
    }
    sR[0][tid] = aA;
    sR[1][tid] = aD;
    sR[2][tid] = aT;
    __syncthreads();
    if (tid == 0) {
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
        for (int j = 0; j < kScalThreads; ++j) { s0 += sR[0][j]; s1 += sR[1][j]; s2 += sR[2][j]; }
        p.pA[i] = s0;
        p.pD[i] = s1;
        p.pT[i] = s2;
    }
}

// dA_log = A * sum over (batch, segment), dD, ddt_bias = sums over (batch, segment)
__global__ void __launch_bounds__(256) ssdb_final(SbKp p) {
    const int64_t h = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (h >= p.H) return;
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
    for (int64_t bk = 0; bk < p.batch * p.nseg; ++bk) {
        s0 += p.pA[bk * p.H + h];
        s1 += p.pD[bk * p.H + h];
        s2 += p.pT[bk * p.H + h];
    }
    if (p.dA_log) p.dA_log[h] = s0 * -expf(p.A_log[h]);
    if (p.dD) p.dD[h] = s1;
    if (p.ddt_bias) p.ddt_bias[h] = s2;
}

// ---------------------------------------------------------------------------
// Mamba-3 trapezoidal backward, after the SSD backward of the shifted state.
// The forward is SSD(sigma) plus, at each step, (gamma_t - sigma_t)(q_t.k_t) x_t
// (its chunk diagonal uses gamma), and its entering state is
// h0' = h0 + c_0 x_prev (x) k_prev with c_t = dt_t (1 - trap_t).

// The entering state's gradient dh0' = dL/dh0 (copied out) and, with the carried
// pair, dx_prev = c_0 dh0' k_prev, dk_prev = c_0 dh0'^T x_prev and
// dc_0 = <dh0', x_prev (x) k_prev>.  One group of 256 per (b, h), fixed-order sums.
__global__ void __launch_bounds__(256) trapb_prev_kernel(SbKp p, const float *dh0p, const uint16_t *x_prev,
                                                        const uint16_t *k_prev, float *dh0, float *dx_prev,
                                                        float *dk_prev, float *dc0) {
    __shared__ float sP[256];
    const int64_t bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
    const int tid = threadIdx.x;
    const float *G = dh0p + bh * p.P * p.N;
    if (dh0)
        for (int64_t i = tid; i < p.P * p.N; i += 256) dh0[bh * p.P * p.N + i] = G[i];
    if (!x_prev) return;
    const int64_t o0 = b * p.L * p.H + h;         // step 0
    const float c0 = p.dt[o0] * (1.0f - p.trap[o0]);
    float part = 0.0f;                            // sum over this thread's rows p of x_prev[p] (G k_prev)[p]
    for (int64_t i = tid; i < p.P; i += 256) {
        float s = 0.0f;
        for (int64_t n = 0; n < p.N; ++n) s = fmaf(G[i * p.N + n], bf(k_prev[bh * p.N + n]), s);
        if (dx_prev) dx_prev[bh * p.P + i] = c0 * s;
        part = fmaf(bf(x_prev[bh * p.P + i]), s, part);
    }
    for (int64_t n = tid; n < p.N; n += 256) {
        float s = 0.0f;
        for (int64_t i = 0; i < p.P; ++i) s = fmaf(G[i * p.N + n], bf(x_prev[bh * p.P + i]), s);
        if (dk_prev) dk_prev[bh * p.N + n] = c0 * s;
    }
    sP[tid] = part;
    __syncthreads();
    if (tid == 0) {
        float tot = 0.0f;
        for (int j = 0; j < 256; ++j) tot += sP[j];
        dc0[bh] = tot;
    }
}

// The chain to the inputs, one thread per (b, t, h).  The walks leave the step's own
// term out of dsig_t = x_t.(G'_t B_t), the gradient of the shifted state's input scale
// sigma_t = gamma_t + c_{t+1}; dgam_t = (q_t.k_t)(dy_t.x_t) is the diagonal, scaled by
// gamma_t alone.  So with da_t = dL/da_t (in dyy),
// dgamma_t = dsig_t + dgam_t and dc_t = dsig_{t-1} (dc_0 at t = 0):
//   ddt = da aval + dgamma trap + dc (1 - trap),  dtrap = (dgamma - dc) dt,  daval = da dt.
__global__ void __launch_bounds__(256) trapb_chain_kernel(SbKp p, const float *dc0, float *ddt, float *daval,
                                                         float *dtrap) {
    const int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (o >= p.batch * p.L * p.H) return;
    const int64_t h = o % p.H, t = (o / p.H) % p.L, b = o / (p.H * p.L);
    const float da = p.dyy[o];
    const float dg = p.dsig[o] + p.dgam[o];
    const float dc = t > 0 ? p.dsig[o - p.H] : (dc0 ? dc0[b * p.H + h] : 0.0f);
    const float dtv = p.dt[o], tr = p.trap[o];
    ddt[o] = fmaf(da, p.aval[o], fmaf(dg, tr, dc * (1.0f - tr)));
    dtrap[o] = (dg - dc) * dtv;
    daval[o] = da * dtv;
}

struct Plan { int64_t nseg, Ls; };
Plan plan(int64_t batch, int64_t L, int64_t H, int64_t N) {
    const int64_t waves = batch * H * (N / 32);
    int64_t nseg = (kTargetWaves + waves - 1) / waves;
    nseg = std::max<int64_t>(1, std::min<int64_t>(nseg, L / kMinSeg));
    nseg = std::max<int64_t>(nseg, (L + kMaxSeg - 1) / kMaxSeg);
    const int64_t Ls = ((L + nseg - 1) / nseg + kQ - 1) / kQ * kQ;
    return Plan{(L + Ls - 1) / Ls, Ls};
}
size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

struct WsLayout { size_t Sseg, Gseg, dec, bnd, dBh, dCh, dyy, dsig, dyx, dgam, hfdot, pA, pD, pT, total; };
// shares: each head's share of dB and dC is kept for the sum over a group's
// heads; with one head per group the walks write dB and dC themselves
WsLayout layout(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t nseg, bool shares) {
    WsLayout w{};
    size_t o = 0;
    const size_t seg = nseg > 1 ? (size_t)(batch * H * nseg * P * N) * 4 : 0;
    w.Sseg = o; o += al256(seg);
    w.Gseg = o; o += al256(seg);
    w.dec = o;  o += al256((size_t)(batch * H * nseg) * 4);
    w.bnd = o;  o += al256((size_t)(batch * H * nseg) * 8);
    const size_t sh = shares ? (size_t)(batch * L * H * N) * 4 : 0;
    w.dBh = o;  o += al256(sh);
    w.dCh = o;  o += al256(sh);
    w.dyy = o;  o += al256((size_t)(batch * L * H) * 4);
    w.dsig = o; o += al256((size_t)(batch * L * H) * 4);
    w.dyx = o;  o += al256((size_t)(batch * L * H) * 4);
    w.dgam = o; o += al256((size_t)(batch * L * H) * 4);
    w.hfdot = o; o += al256((size_t)(batch * H) * 4);
    w.pA = o;   o += al256((size_t)(batch * nseg * H) * 4);
    w.pD = o;   o += al256((size_t)(batch * nseg * H) * 4);
    w.pT = o;   o += al256((size_t)(batch * nseg * H) * 4);
    w.total = o;
    return w;
}

template <int P, int N>
void launch_pn(const SbKp &p, hipStream_t s) {
    const unsigned bh = (unsigned)(p.batch * p.H);
    if (p.nseg > 1) {
        hipLaunchKernelGGL((ssdb_walk_f<P, N, true>), dim3(bh * (unsigned)(p.nseg - 1)), dim3(64 * (N / 32)), 0, s, p);
        hipLaunchKernelGGL((ssdb_walk_r1<P, N, true>), dim3(bh * (unsigned)(p.nseg - 1)), dim3(64 * (N / 32)), 0, s, p);
        const int64_t tot = p.batch * p.H * p.P * p.N;
        hipLaunchKernelGGL(ssdb_pass_f, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, p);
        hipLaunchKernelGGL(ssdb_pass_r, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, p);
        hipLaunchKernelGGL(ssdb_bnd, dim3(bh * (unsigned)(p.nseg - 1)), dim3(kBndThreads), 0, s, p);
    }
    // R2 first: the trapezoidal form's dq, dk corrections in F and R1 use its dy.x
    hipLaunchKernelGGL((ssdb_walk_r2<P, N>), dim3(bh * (unsigned)p.nseg), dim3(64 * (P / 16)), 0, s, p);
    hipLaunchKernelGGL((ssdb_walk_f<P, N, false>), dim3(bh * (unsigned)p.nseg), dim3(64 * (N / 32)), 0, s, p);
    hipLaunchKernelGGL((ssdb_walk_r1<P, N, false>), dim3(bh * (unsigned)p.nseg), dim3(64 * (N / 32)), 0, s, p);
    if (p.G != p.H) {
        const int64_t nr = p.batch * p.L * p.G * p.N;
        hipLaunchKernelGGL(ssdb_reduce_heads, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, s, p);
    }
    hipLaunchKernelGGL(ssdb_scal, dim3((unsigned)(p.batch * p.nseg * p.H)), dim3(kScalThreads), 0, s, p);
    hipLaunchKernelGGL(ssdb_final, dim3((unsigned)((p.H + 255) / 256)), dim3(256), 0, s, p);
}

template <int P>
void launch_p(const SbKp &p, hipStream_t s) {
    if (p.N == 32) launch_pn<P, 32>(p, s);
    else if (p.N == 64) launch_pn<P, 64>(p, s);
    else launch_pn<P, 128>(p, s);
}

}  // namespace

size_t ssd_trap_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state) {
    const Plan pl = plan(batch, L, nheads, d_state);
    const size_t st = al256((size_t)(batch * nheads * headdim * d_state) * 4);
    return layout(batch, L, nheads, headdim, d_state, pl.nseg, false).total + 2 * st +
           al256((size_t)(batch * nheads) * 4);
}

size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                               int64_t ngroups) {
    const Plan pl = plan(batch, L, nheads, d_state);
    return layout(batch, L, nheads, headdim, d_state, pl.nseg, ngroups != nheads).total;
}

namespace {
// the parameter block and workspace views of one backward call
SbKp make_params(const SsdBwdArgs &a) {
    SbKp p{};
    p.x = static_cast<const uint16_t *>(a.x);
    p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log;
    p.B = static_cast<const uint16_t *>(a.B);
    p.C = static_cast<const uint16_t *>(a.C);
    p.D = a.D; p.h0 = a.h0; p.dy = a.dy; p.dhf = a.dh_final;
    p.dx = a.dx; p.ddt = a.ddt; p.dB = a.dB; p.dC = a.dC; p.dA_log = a.dA_log; p.dD = a.dD;
    p.ddt_bias = a.ddt_bias; p.dh0 = a.dh0;
    p.batch = a.batch; p.L = a.L; p.H = a.nheads; p.P = a.headdim; p.N = a.d_state; p.G = a.ngroups;
    p.mode = (int)(a.flags & 0x3u);
    const Plan pl = plan(a.batch, a.L, a.nheads, a.d_state);
    p.nseg = pl.nseg;
    p.Ls = pl.Ls;
    const WsLayout w = layout(a.batch, a.L, a.nheads, a.headdim, a.d_state, pl.nseg, a.ngroups != a.nheads);
    char *ws = static_cast<char *>(a.workspace);
    p.Sseg = reinterpret_cast<float *>(ws + w.Sseg);
    p.Gseg = reinterpret_cast<float *>(ws + w.Gseg);
    p.dec = reinterpret_cast<float *>(ws + w.dec);
    p.dBh = a.ngroups == a.nheads ? a.dB : reinterpret_cast<float *>(ws + w.dBh);
    p.dCh = a.ngroups == a.nheads ? a.dC : reinterpret_cast<float *>(ws + w.dCh);
    p.dyy = reinterpret_cast<float *>(ws + w.dyy);
    p.dsig = reinterpret_cast<float *>(ws + w.dsig);
    p.dyx = reinterpret_cast<float *>(ws + w.dyx);
    p.dgam = reinterpret_cast<float *>(ws + w.dgam);
    p.hfdot = reinterpret_cast<float *>(ws + w.hfdot);
    p.bnd = reinterpret_cast<double *>(ws + w.bnd);
    p.pA = reinterpret_cast<float *>(ws + w.pA);
    p.pD = reinterpret_cast<float *>(ws + w.pD);
    p.pT = reinterpret_cast<float *>(ws + w.pT);
    return p;
}
void launch_walks(const SbKp &p, hipStream_t stream) {
    if (p.P == 32) launch_p<32>(p, stream);
    else if (p.P == 64) launch_p<64>(p, stream);
    else launch_p<128>(p, stream);
}
}  // namespace

hipError_t launch_ssd_bwd(const SsdBwdArgs &a, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "ssdb_walk_f";
    const SbKp p = make_params(a);
    launch_walks(p, stream);
    return hipGetLastError();
}

hipError_t launch_ssd_trap_bwd(const SsdTrapBwdArgs &t, hipStream_t stream, const char **kernel_name) {
    // the SSD backward of the shifted state: B = k, C = q, one group per head
    const Plan pl = plan(t.batch, t.L, t.nheads, t.d_state);
    char *ws = static_cast<char *>(t.workspace);
    const size_t base = layout(t.batch, t.L, t.nheads, t.headdim, t.d_state, pl.nseg, false).total;
    const size_t st = al256((size_t)(t.batch * t.nheads * t.headdim * t.d_state) * 4);
    float *h0p = reinterpret_cast<float *>(ws + base);
    float *dh0p = reinterpret_cast<float *>(ws + base + st);
    float *dc0 = reinterpret_cast<float *>(ws + base + 2 * st);
    const float *h0 = t.h0;
    if (t.x_prev) {
        *kernel_name = "ssd_trap_h0_kernel";
        const hipError_t e = launch_ssd_trap_h0(t.x_prev, t.k_prev, t.dt, t.trap, t.h0, h0p, t.batch, t.L, t.nheads,
                                                t.headdim, t.d_state, stream);
        if (e != hipSuccess) return e;
        h0 = h0p;
    }
    SsdBwdArgs a{t.x, t.dt, nullptr, nullptr, t.k, t.q, t.D, h0, t.dy, t.dh_final,
                 t.dx, nullptr, t.dk, t.dq, nullptr, t.dD, nullptr, dh0p,
                 t.batch, t.L, t.nheads, t.headdim, t.d_state, t.nheads, 0x1u, t.workspace};
    SbKp p = make_params(a);
    p.aval = t.a;
    p.trap = t.trap;
    *kernel_name = "ssdb_walk_f";
    launch_walks(p, stream);
    *kernel_name = "trapb_prev_kernel";
    hipLaunchKernelGGL(trapb_prev_kernel, dim3((unsigned)(t.batch * t.nheads)), dim3(256), 0, stream, p, dh0p,
                       static_cast<const uint16_t *>(t.x_prev), static_cast<const uint16_t *>(t.k_prev), t.dh0,
                       t.dx_prev, t.dk_prev, dc0);
    *kernel_name = "trapb_chain_kernel";
    const int64_t n = t.batch * t.L * t.nheads;
    hipLaunchKernelGGL(trapb_chain_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p,
                       t.x_prev ? dc0 : nullptr, t.ddt, t.da, t.dtrap);
    return hipGetLastError();
}

}  // namespace ssm
