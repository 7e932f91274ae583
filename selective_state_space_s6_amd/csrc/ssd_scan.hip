// ssd_scan.hip -- Mamba-2 state-space-dual (SSD) forward scan, gfx950.
//
// Implements the scalar-A-per-head recurrence of builderforce-memory-engine
// ssd.js (header comment, ssd_chunk_forward) by the chunked decomposition that
// mamba-rs 0.2.1 mamba3_gpu.rs step F6 launches as separate kernels (dA
// cumsum, chunk state, state passing, chunk scan, final-state writeback).
//
// The sequence of every (batch, head) is cut into a few long segments so that
// enough work groups exist to fill the chip; inside a segment the state is
// carried on chip from one 32-step chunk to the next:
//
//   ssd_state_kernel   per (batch, segment, head), all segments but the last:
//                      the segment's own final state from a zero start (D2 and
//                      D3 inside the segment) and its total decay e^{sum a}
//   ssd_pass_kernel    per (batch, head): the state entering every segment,
//                      S_in[k+1] = e^{sum a over k} S_in[k] + S_local[k]  (D3)
//   ssd_scan_kernel    per (batch, segment, head): from S_in[k], per chunk
//     D1  delta = softplus(dt + dt_bias), a = delta*A_h, cs = cumsum(a), sigma
//     D4  y_intra = ((C B^T) o L) X with L[t,s] = e^{cs_t-cs_s} sigma_s, s <= t
//     D5  y += e^{cs_t} C_t S + D x_t
//     D2  S <- e^{cs_end} S + B^T (w o X), w_s = e^{cs_end-cs_s} sigma_s  (D3)
//     and after the last chunk of the last segment S is h_final.
//
// A work group holds one head: headdim/16 waves, each owning 16 head channels
// and keeping their N x 16 slice of the fp32 state in MFMA accumulators.  The
// chunk's C.B^T and decay mask (D4) are computed once per group, split over
// the first waves, and shared through LDS.  Every contraction is a bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with fp32 accumulation.  x, B, C are bf16 and
// exact; products formed in fp32 (w o X, the masked C.B^T, the state) are split
// into bf16 hi + lo parts and contracted twice, keeping ~16 mantissa bits.
// Chunks are double-buffered in LDS; the loads of chunk j+2 are in flight
// while chunk j is computed.
#include "device_common.hpp"
#include "launchers.hpp"
#include <algorithm>

namespace ssm {
namespace {

// bf16 operands travel as raw 16-bit patterns in 32-bit lanes and are
// reinterpreted as whole vectors at the MFMA: element-wise access to __bf16
// vectors is avoided on purpose.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 32;              // steps per chunk
constexpr int kCUs = 256;           // compute units of the chip
constexpr int kWavesPerCU = 12;     // resident waves per CU at the kernels' register use (3 per SIMD)
constexpr int kMaxSeg = 64;         // at most this many segments (bounds the workspace)
constexpr int kMinSeg = 256;        // shortest segment worth a state round trip

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// two fp32 -> two bf16 (round to nearest even), low half = a
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// v = hi + lo with hi, lo bf16; returns {hi pair, lo pair}
__device__ __forceinline__ uint2 split_bf16(float a, float b) {
    const uint32_t hi = pack_bf16(a, b);
    return make_uint2(hi, pack_bf16(a - lo_f(hi), b - hi_f(hi)));
}

// A lane's 32-bit byte offset, re-read where it is used: the empty asm keeps the
// compiler from hoisting its zero extension out of a loop, so that base (uniform)
// + offset stays the global instructions' SGPR-base form instead of a 64-bit add
// per access
__device__ __forceinline__ uint32_t lane_off(uint32_t o) {
    asm volatile("" : "+v"(o));
    return o;
}

// Word 3 of a raw buffer resource on gfx9-family chips (gfx950 included): 32-bit data
// format, no swizzle, no index stride; with stride 0 an access whose offset is at or past
// the record count is dropped (stores) or reads zero (loads)
constexpr int kBufWord3 = 0x00020000;

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i
// names a row of 4 consecutive 16-bit elements and receives element (i % 4) of
// rows i/4, i/4 + 4, i/4 + 8, i/4 + 12.  Pointing row i at (step sb + i/4,
// column cb + 4*(i%4)) of a row-major [step][column] tile hands lane i the four
// steps sb..sb+3 of column cb + i: the layout an MFMA operand needs when the
// time step is the contraction index.
__device__ __forceinline__ uint2 tr_read(const uint16_t *tile, int pitch, int sb, int cb, int lane) {
    const int i = lane & 15;
    const uint16_t *a = tile + (sb + (i >> 2)) * pitch + cb + 4 * (i & 3);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(a));
    return __builtin_bit_cast(uint2, v);
}

struct SsdKp {
    const uint16_t *x; const float *dt; const float *dt_bias; const float *A_log;
    const uint16_t *B; const uint16_t *C; const float *D; float *y;
    const float *h0; float *h_final;
    float *ws_state;    // (batch, H, nseg, P, N): local, then entering, segment states
    float *ws_decay;    // (batch, H, nseg): e^{sum of a} over a segment
    int64_t batch, L, H, P, N, G;
    int64_t Ls, nseg;   // segment length (a multiple of kT) and count
    int mode;           // 0 ZOH, 1 DT, 2 ONE
    // Mamba-3 trapezoidal form (when trap is set): dt is used as given, a_t =
    // dt_t aval_t, the input scale is gamma_t + dt_{t+1} (1 - trap_{t+1}) and the
    // diagonal of the intra-chunk matrix uses gamma_t = trap_t dt_t
    const float *aval, *trap;   // (batch, L, H)
};


// per-chunk scalars in LDS
struct Scal {
    float cs[kT];    // inclusive cumulative sum of a from the chunk start
    float ecs[kT];   // e^{cs_t}
    float sig[kT];   // input scale
    float gam[kT];   // input scale of the step's own output (differs from sig in the trapezoidal form)
    float w[kT];     // e^{cs_end - cs_s} sigma_s
    float end;       // e^{cs_end}
};

// D1 for one chunk, by one wave (lanes 0..31 hold steps 0..31).
// Trapezoidal inputs of one step (used when the kernel runs that form).
struct TrapIn { float av, tr, dtn, trn; bool nvalid; };

__device__ __forceinline__ void chunk_scalars(Scal &sc, float dtv, bool valid, float bias, float A,
                                              int mode, int lane, const TrapIn *ti = nullptr) {
    float a = 0.0f, sg = 0.0f, gm = 0.0f;
    if (valid) {
        if (ti) {
            a = dtv * ti->av;
            gm = ti->tr * dtv;
            sg = gm + (ti->nvalid ? ti->dtn * (1.0f - ti->trn) : 0.0f);
        } else {
            const float dl = softplus(dtv + bias);
            a = dl * A;
            if (mode == 1) sg = dl;
            else if (mode == 0) sg = (a == 0.0f) ? dl : dl * (expm1f(a) / a);
            else sg = 1.0f;
            gm = sg;
        }
    }
    const float v = scan32(a);
    const float cend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    if (lane < kT) {
        sc.cs[lane] = v;
        sc.ecs[lane] = __expf(v);
        sc.sig[lane] = sg;
        sc.gam[lane] = gm;
        sc.w[lane] = __expf(cend - v) * sg;
    }
    if (lane == 0) sc.end = __expf(cend);
}

// x tile row pitch (bf16) for P head channels in the scan kernel: the row
// stride in dwords is 24, 36 or 12 (mod 64), so the four rows that 16 lanes of
// a transposed read take (8 dwords each) fall on distinct banks.  The 32 lanes
// served per cycle still meet on a few banks (2-way); the state kernel, whose
// tiles see only transposed reads, uses the conflict-free pitch P + 16.
constexpr int x_pitch(int P) { return P == 32 ? 48 : P == 64 ? 72 : 152; }

// LDS and register staging of one chunk of x, B (and C), dt for a work group
// of NW waves per head holding HPW consecutive heads h.. of one group (B and C
// staged once for them; x and dt per head, each by that head's threads).  Loads are unconditional so they stay in
// flight across a chunk.  Addresses are a uniform base (the chunk's first row)
// plus a 32-bit per-thread offset; a chunk that crosses L clamps its step
// index into the tensors (rows past L never contribute: their sigma and w are
// 0 and their outputs are not stored).
template <int NMAX, int NW, bool WITH_C, int NS = 1, bool TRAP = false, bool ROWS8 = false, int HPW = 1>
struct Stager {
    static constexpr int NTHR = 64 * NW * HPW;
    static constexpr int P = 16 * NW;
    // B/C and x row pitches (bf16).  ROWS8: the tiles are read only by
    // transposed reads in which 32 lanes take 8 consecutive rows, 8 dwords each
    // (ds_read_b64_tr_b16 serves 32 lanes per cycle): a row stride of an odd
    // multiple of 8 dwords puts them on distinct banks of the 64
    static constexpr int BCP = ROWS8 ? NMAX + 16 : NMAX == 64 ? 72 : 2 * (NMAX / 2 + 12);
    static constexpr int XP = ROWS8 ? P + 16 : x_pitch(P);
    static constexpr int LDN = NMAX / 8;                // 16-byte pieces per B/C row
    static constexpr int PER_T = kT * LDN / NTHR;       // B (and C) pieces per thread
    static constexpr int SB_STEP = NTHR / LDN;          // steps between pieces i, i+1
    static constexpr int XPR = P / 8;                   // 16-byte pieces per x row
    static_assert(PER_T >= 1 && kT * LDN % NTHR == 0 && NTHR % LDN == 0, "B/C pieces must divide evenly");
    static_assert(kT * XPR == 64 * NW, "one x piece per thread of each head");

    // NS register stages: a chunk is loaded NS chunks before it is staged to LDS
    u32x4 rB[NS][PER_T], rC[NS][PER_T], rX[NS];
    float rdt[NS];
    TrapIn rtp[TRAP ? NS : 1];      // trapezoidal inputs of this thread's dt step
    const uint16_t *Bb, *Cb, *Xb;   // step 0 of this (batch, group) / (batch, head)
    const float *Db, *Ab, *Tb;
    uint32_t colB;                  // this thread's B/C column (clamped into the state)
    int sB, nB, sX, cX, sD, xo;     // xo: this thread's head's x tile in LDS
    uint32_t oB, oX;                // byte offsets of this thread's B/C and x pieces in a chunk
    int64_t rowBC, rowX, H, L;

    __device__ __forceinline__ void init(const SsdKp &p, int64_t b, int64_t h, int64_t g, int N, int tid) {
        rowBC = p.G * p.N;
        rowX = p.H * p.P;
        H = p.H;
        L = p.L;
        // the thread's head in the group: uniform over a wave (an SGPR), so the
        // head's base pointers stay scalar
        const int xh = HPW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / (64 * NW));
        const int tx = tid - xh * 64 * NW;
        sB = tid / LDN;
        nB = (tid % LDN) * 8;
        sX = tx / XPR;
        cX = (tx % XPR) * 8;
        sD = tid & 31;
        xo = xh * kT * XP;
        colB = (uint32_t)min(nB, N - 8);
        oB = ((uint32_t)sB * (uint32_t)rowBC + colB) * 2u;
        oX = ((uint32_t)sX * (uint32_t)rowX + (uint32_t)cX) * 2u;
        Bb = p.B + (b * p.L * p.G + g) * p.N;
        Cb = p.C + (b * p.L * p.G + g) * p.N;
        Xb = p.x + (b * p.L * p.H + h + xh) * p.P;
        Db = p.dt + b * p.L * p.H + h + xh;
        Ab = p.aval ? p.aval + b * p.L * p.H + h + xh : nullptr;
        Tb = p.trap ? p.trap + b * p.L * p.H + h + xh : nullptr;
    }
    // a, trap of step t0 + i and dt, trap of step t0 + i + 1 (clamped into the
    // sequence; nvalid marks whether that next step exists)
    template <int S>
    __device__ __forceinline__ void load_trap(int64_t t0, int i) {
        const int64_t t = min(t0 + i, L - 1), tn = t0 + i + 1;
        const int64_t tc = min(tn, L - 1);
        rtp[S].av = Ab[t * H];
        rtp[S].tr = Tb[t * H];
        rtp[S].dtn = Db[tc * H];
        rtp[S].trn = Tb[tc * H];
        rtp[S].nvalid = tn < L;
    }
    template <int S>
    __device__ __forceinline__ void load(int64_t t0) {
        const uint16_t *Bu = Bb + t0 * rowBC, *Cu = Cb + t0 * rowBC, *Xu = Xb + t0 * rowX;
        const float *Du = Db + t0 * H;
        if (t0 + kT <= L) {
            // uniform row base + the lane's 32-bit byte offset (SGPR-base loads)
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                rB[S][i] = *reinterpret_cast<const u32x4 *>(
                    reinterpret_cast<const char *>(Bu + SB_STEP * i * rowBC) + lane_off(oB));
                if constexpr (WITH_C)
                    rC[S][i] = *reinterpret_cast<const u32x4 *>(
                        reinterpret_cast<const char *>(Cu + SB_STEP * i * rowBC) + lane_off(oB));
            }
            rX[S] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(Xu) + lane_off(oX));
            rdt[S] = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(Du) +
                                                      lane_off((uint32_t)sD * (uint32_t)H * 4u));
            if constexpr (TRAP) load_trap<S>(t0, sD);
        } else {
            const int last = (int)(L - 1 - t0);   // last valid step of the chunk
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const uint32_t o = (uint32_t)(min(sB + SB_STEP * i, last) * rowBC) + colB;
                rB[S][i] = *reinterpret_cast<const u32x4 *>(Bu + o);
                if constexpr (WITH_C) rC[S][i] = *reinterpret_cast<const u32x4 *>(Cu + o);
            }
            rX[S] = *reinterpret_cast<const u32x4 *>(Xu + (uint32_t)(min(sX, last) * rowX + cX));
            rdt[S] = Du[(uint32_t)(min(sD, last) * H)];
            if constexpr (TRAP) load_trap<S>(t0, min(sD, last));
        }
    }
    template <int S>
    __device__ __forceinline__ void store(uint16_t *Bs, uint16_t *Cs, uint16_t *Xs) {
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int o = (sB + SB_STEP * i) * BCP + nB;
            *reinterpret_cast<u32x4 *>(&Bs[o]) = rB[S][i];
            if constexpr (WITH_C) *reinterpret_cast<u32x4 *>(&Cs[o]) = rC[S][i];
        }
        *reinterpret_cast<u32x4 *>(&Xs[xo + sX * XP + cX]) = rX[S];
    }
};

// Decay-weighted inputs w_s x[s][p] of one wave's 16 channels as hi/lo bf16
// into the wave's own [step][channel] tiles (row pitch 16: the four rows of a
// transposed read are 32 consecutive dwords, so no bank is hit twice).
constexpr int WP = 16;
template <int XP>
__device__ __forceinline__ void weighted_x(const uint16_t *Xs, int p0, const float *w, uint16_t *Wh,
                                           uint16_t *Wl, int lane) {
    const int s = lane >> 1, c8 = (lane & 1) * 8;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(&Xs[s * XP + p0 + c8]);
    const float ws = w[s];
    u32x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint2 sp = split_bf16(ws * lo_f(v[i]), ws * hi_f(v[i]));
        hi[i] = sp.x;
        lo[i] = sp.y;
    }
    *reinterpret_cast<u32x4 *>(&Wh[s * WP + c8]) = hi;
    *reinterpret_cast<u32x4 *>(&Wl[s * WP + c8]) = lo;
    // the same wave reads these rows back (transposed): LDS operations of one
    // wave complete in order, and this keeps the compiler from moving the reads
    // above the writes
    asm volatile("" ::: "memory");
}

// D2+D3 for one wave: S <- e^{cs_end} S + B^T (w o X); A = B^T via transposed reads
template <int NT, int BCP>
__device__ __forceinline__ void state_update(f32x4 (&S)[NT], const uint16_t *B_, const uint16_t *Wh,
                                             const uint16_t *Wl, float e, int N, int lane) {
    const int q = lane >> 4;
    const uint2 wh0 = tr_read(Wh, WP, q * 8, 0, lane);
    const uint2 wh1 = tr_read(Wh, WP, q * 8 + 4, 0, lane);
    const uint2 wl0 = tr_read(Wl, WP, q * 8, 0, lane);
    const uint2 wl1 = tr_read(Wl, WP, q * 8 + 4, 0, lane);
    const u32x4 Whf{wh0.x, wh0.y, wh1.x, wh1.y}, Wlf{wl0.x, wl0.y, wl1.x, wl1.y};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (nt * 16 >= N) break;
        S[nt] *= e;
        const uint2 a0 = tr_read(B_, BCP, q * 8, nt * 16, lane);
        const uint2 a1 = tr_read(B_, BCP, q * 8 + 4, nt * 16, lane);
        const u32x4 Af{a0.x, a0.y, a1.x, a1.y};
        S[nt] = mfma16(Af, Whf, S[nt]);
        S[nt] = mfma16(Af, Wlf, S[nt]);
    }
}

// D2+D3 for one wave with the weighted inputs as B operands in registers, K
// slot q*8+i <-> step q*4+i (i < 4) and 16+q*4+(i-4) (i >= 4); the A operand
// B^T is read transposed in the same step order, so the 32 lanes of one read
// cover 8 consecutive rows
template <int NT, int BCP>
__device__ __forceinline__ void state_update_regs(f32x4 (&S)[NT], const uint16_t *B_, u32x4 Whf, u32x4 Wlf,
                                                  float e, int N, int lane) {
    const int q = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (nt * 16 >= N) break;
        S[nt] *= e;
        const uint2 a0 = tr_read(B_, BCP, q * 4, nt * 16, lane);
        const uint2 a1 = tr_read(B_, BCP, 16 + q * 4, nt * 16, lane);
        const u32x4 Af{a0.x, a0.y, a1.x, a1.y};
        S[nt] = mfma16(Af, Whf, S[nt]);
        S[nt] = mfma16(Af, Wlf, S[nt]);
    }
}

// The weighted inputs w_s x[s][p] of one wave's 16 channels for the steps of
// that K order, as hi + lo B operands, from the x tile (transposed reads) and
// the step weights
template <int XP>
__device__ __forceinline__ void weighted_x_regs(const uint16_t *Xs, int p0, const float *w, int lane,
                                                u32x4 &Whf, u32x4 &Wlf) {
    const int q = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const uint2 xv = tr_read(Xs, XP, tt * 16 + q * 4, p0, lane);
        const float4 w4 = *reinterpret_cast<const float4 *>(&w[tt * 16 + q * 4]);
        const uint2 u0 = split_bf16(w4.x * lo_f(xv.x), w4.y * hi_f(xv.x));
        const uint2 u1 = split_bf16(w4.z * lo_f(xv.y), w4.w * hi_f(xv.y));
        Whf[2 * tt] = u0.x; Whf[2 * tt + 1] = u1.x;
        Wlf[2 * tt] = u0.y; Wlf[2 * tt + 1] = u1.y;
    }
}

// work index -> (b, segment, h); heads of one (batch, segment) are consecutive,
// so the groups that share B and C rows land on one XCD
struct Work {
    int64_t b, k, h;
    __device__ __forceinline__ Work(int64_t work, int64_t H, int64_t nseg)
        : b(work / (H * nseg)), k((work / H) % nseg), h(work % H) {}
};

// ---- the segment's own final state (zero start) and total decay; every
// segment but the last, all of whose chunks are whole.
//   S_local[p][n] = sum_s e^{sum_{r > s} a_r} sigma_s x_s[p] B_s[n]
// The segment is walked backwards, so the weight of step s is one exp of the
// running suffix sum of a (same-signed terms, no cancellation) and the state
// needs no rescaling between chunks; the contraction over s is a plain GEMM.
// Chunks are loaded NS = 2 chunks ahead (two register stages keep the kernel
// within 128 registers, four groups of four waves per compute unit).
template <int NS, int I, typename F>
__device__ __forceinline__ void unroll_stages(F &&f) {
    if constexpr (I < NS) {
        f(std::integral_constant<int, I>{});
        unroll_stages<NS, I + 1>(f);
    }
}

// HPW heads of one group per work group (NW waves each): B is staged once for
// them, x and the weights per head.
template <int NMAX, bool EXACT, int NW, bool TRAP, int HPW>
__global__ void __launch_bounds__(64 * NW * HPW)
ssd_state_kernel(SsdKp p) {
    constexpr int NS = 2;
    using St = Stager<NMAX, NW, false, NS, TRAP, true, HPW>;
    constexpr int NT = NMAX / 16;
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kT * St::BCP];
    __shared__ __attribute__((aligned(16))) uint16_t Xs[2][HPW * kT * St::XP];
    __shared__ __attribute__((aligned(16))) float wsc[2][HPW][kT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int hl = wid / NW, wh = wid % NW;                      // head in the group, wave in the head
    const int c16 = lane & 15, q = lane >> 4;
    const int64_t nseg1 = p.nseg - 1;
    const Work wk(xcd_swizzle(blockIdx.x, p.batch * nseg1 * (p.H / HPW)), p.H / HPW, nseg1);
    const int64_t h0 = wk.h * HPW, h = h0 + hl;
    const int64_t g = h0 * p.G / p.H;
    const int p0 = wh * 16;
    const int N = EXACT ? NMAX : (int)p.N;
    const float A = p.A_log ? -expf(p.A_log[h]) : 0.0f;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;

    f32x4 S[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) S[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    St st;
    st.init(p, wk.b, h0, g, N, tid);
    st.sD = kT - 1 - (tid & 31);                           // dt lanes in reverse step order
    const int64_t nch = p.Ls / kT;
    const int64_t tlast = wk.k * p.Ls + (nch - 1) * kT;   // first step of the last chunk
    // weights of one chunk from its dt (each head's wave 0; lane i holds step
    // 31 - i, so the lane-order prefix sum is the step-order suffix sum); R is
    // the sum of a over the later steps of the segment, kept by that wave
    float R = 0.0f;
    auto weights = [&](float *w, float dtv, const TrapIn &ti) __attribute__((always_inline)) {
        float a, sg;
        if constexpr (TRAP) {
            a = dtv * ti.av;
            sg = ti.tr * dtv + (ti.nvalid ? ti.dtn * (1.0f - ti.trn) : 0.0f);
        } else {
            const float dl = softplus(dtv + bias);
            a = dl * A;
            if (p.mode == 1) sg = dl;
            else if (p.mode == 0) sg = (a == 0.0f) ? dl : dl * (expm1f(a) / a);
            else sg = 1.0f;
        }
        const float v = scan32(a);                     // sum of a over steps >= this step
        if (lane < kT) w[kT - 1 - lane] = __expf(R + (v - a)) * sg;
        R += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    };

    unroll_stages<NS, 0>([&](auto sTag) __attribute__((always_inline)) {
        constexpr int S_ = decltype(sTag)::value;
        if (S_ < nch) st.template load<S_>(tlast - S_ * kT);
    });
    st.template store<0>(Bs[0], nullptr, Xs[0]);
    if (wh == 0) weights(wsc[0][hl], st.rdt[0], st.rtp[0]);
    if (NS < nch) st.template load<0>(tlast - NS * kT);
    __syncthreads();

    // chunk c (c = 0 is the last chunk of the segment) is in register stage c % NS
    for (int64_t c0 = 0; c0 < nch; c0 += NS) {
        unroll_stages<NS, 0>([&](auto sTag) __attribute__((always_inline)) {
            constexpr int S_ = decltype(sTag)::value;
            const int64_t c = c0 + S_;
            if (c >= nch) return;
            const int buf = (int)(c & 1);
            u32x4 Whf, Wlf;
            weighted_x_regs<St::XP>(Xs[buf] + hl * kT * St::XP, p0, wsc[buf][hl], lane, Whf, Wlf);
            state_update_regs<NT, St::BCP>(S, Bs[buf], Whf, Wlf, 1.0f, N, lane);
            if (c + 1 < nch) {
                constexpr int SN = (S_ + 1) % NS;
                st.template store<SN>(Bs[buf ^ 1], nullptr, Xs[buf ^ 1]);
                if (wh == 0) weights(wsc[buf ^ 1][hl], st.rdt[SN], st.rtp[TRAP ? SN : 0]);
                if (c + 1 + NS < nch) st.template load<SN>(tlast - (c + 1 + NS) * kT);
            }
            __syncthreads();
        });
    }

    const int64_t slot = (wk.b * p.H + h) * p.nseg + wk.k;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (nt * 16 >= N) break;
        float *dst = p.ws_state + (slot * p.P + p0 + c16) * p.N + nt * 16 + q * 4;
        *reinterpret_cast<float4 *>(dst) = make_float4(S[nt][0], S[nt][1], S[nt][2], S[nt][3]);
    }
    if (wh == 0 && lane == 0) p.ws_decay[slot] = __expf(R);
}

// ---- D3 across segments: the state entering each segment, in place of the
// segment-local states.  One thread per 4 consecutive (p, n) of one (b, h).
__global__ void __launch_bounds__(256)
ssd_pass_kernel(SsdKp p) {
    const int64_t per = p.P * p.N / 4;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= p.batch * p.H * per) return;
    const int64_t bh = i / per, e = i % per;
    float4 S = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (p.h0) S = reinterpret_cast<const float4 *>(p.h0)[bh * per + e];
    float4 *ws = reinterpret_cast<float4 *>(p.ws_state) + bh * p.nseg * per + e;
    for (int64_t k = 0; k + 1 < p.nseg; ++k) {
        const float4 loc = ws[k * per];
        const float d = p.ws_decay[bh * p.nseg + k];
        ws[k * per] = S;
        S = make_float4(fmaf(d, S.x, loc.x), fmaf(d, S.y, loc.y), fmaf(d, S.z, loc.z), fmaf(d, S.w, loc.w));
    }
    ws[(p.nseg - 1) * per] = S;
}

// ---- outputs of one segment from the state entering it
template <int NMAX, bool EXACT, int NW, bool TRAP>
__global__ void __launch_bounds__(64 * NW)
ssd_scan_kernel(SsdKp p) {
    using St = Stager<NMAX, NW, true, 1, TRAP>;
    constexpr int NT = NMAX / 16;          // state tiles (16 states each) per wave
    constexpr int BCP = St::BCP, XP = St::XP;
    // Once a chunk's C tile has been consumed (after the first barrier of the
    // chunk) it holds the waves' weighted inputs, when they fit; that keeps
    // three groups of four waves resident per CU.
    constexpr bool W_IN_C = NW * 2 * kT * WP <= kT * BCP;
    constexpr int WSEP = W_IN_C ? 1 : NW;
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kT * BCP];
    __shared__ __attribute__((aligned(16))) uint16_t Cs[2][kT * BCP];
    __shared__ __attribute__((aligned(16))) uint16_t Xs[2][kT * XP];
    __shared__ __attribute__((aligned(16))) uint16_t Wsep[WSEP][2 * kT * WP];
    // masked C.B^T of the chunk as the A operand of M X: [time tile][hi, lo][lane]
    __shared__ __attribute__((aligned(16))) u32x4 Ms[2][2][64];
    __shared__ Scal scal[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int c16 = lane & 15, q = lane >> 4;
    const Work wk(xcd_swizzle(blockIdx.x, p.batch * p.nseg * p.H), p.H, p.nseg);
    const int64_t g = wk.h * p.G / p.H;
    const int p0 = wid * 16;                 // this wave's first head channel
    const int N = EXACT ? NMAX : (int)p.N;   // compile-time when the state size is exact
    const float A = p.A_log ? -expf(p.A_log[wk.h]) : 0.0f;
    const float bias = p.dt_bias ? p.dt_bias[wk.h] : 0.0f;
    const float Dh = p.D ? p.D[wk.h] : 0.0f;
    const int64_t rowX = p.H * p.P;
    float *Yg = p.y + (wk.b * p.L * p.H + wk.h) * p.P + p0;
    const uint32_t ylane = (uint32_t)(q * 4 * rowX + c16) * 4u;   // byte offset of the lane's element

    // state slice S[n][p] for n < N, p in this wave's 16 channels, in the MFMA
    // output layout: tile nt, lane (column c16, rows q*4 .. q*4+3)
    const float *Sin = p.nseg > 1 ? p.ws_state + ((wk.b * p.H + wk.h) * p.nseg + wk.k) * p.P * p.N
                                  : (p.h0 ? p.h0 + (wk.b * p.H + wk.h) * p.P * p.N : nullptr);
    f32x4 S[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        S[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (Sin && nt * 16 < N) {
            const float4 v = *reinterpret_cast<const float4 *>(Sin + (p0 + c16) * p.N + nt * 16 + q * 4);
            S[nt] = f32x4{v.x, v.y, v.z, v.w};
        }
    }

    St st;
    st.init(p, wk.b, wk.h, g, N, tid);
    const int64_t tb = wk.k * p.Ls;
    const int64_t te = min(tb + p.Ls, p.L);
    const int64_t nchunks = (te - tb + kT - 1) / kT;
    st.template load<0>(tb);
    st.template store<0>(Bs[0], Cs[0], Xs[0]);
    if (wid == NW - 1)
        chunk_scalars(scal[0], st.rdt[0], tb + (lane & 31) < p.L && lane < kT, bias, A, p.mode, lane,
                      TRAP ? &st.rtp[0] : nullptr);
    if (nchunks > 1) st.template load<0>(tb + kT);
    {
        // the 8 y stores of a chunk, issued here with a record count of 0 (the hardware drops
        // every one): the loop is entered with stores behind the prefetch loads, as from its
        // own back edge, so the compiler's wait at the top of the loop can leave them in flight
        const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(Yg + tb * rowX, 0, 0, kBufWord3);
#pragma unroll
        for (int r = 0; r < 8; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(0u, yr, (int)(ylane + (uint32_t)(r * rowX) * 4u), 0, 0);
    }
    __syncthreads();

    for (int64_t j = 0; j < nchunks; ++j) {
        const int buf = (int)(j & 1);
        const int64_t t0 = tb + j * kT;
        const uint16_t *B_ = Bs[buf], *C_ = Cs[buf], *X_ = Xs[buf];
        const Scal &sc = scal[buf];

        // Stage chunk j+1 (loaded during chunk j-1) into the buffers chunk j-1
        // used, which its closing barrier freed, and start loading chunk j+2,
        // which then has a whole chunk to arrive.  The last wave takes the next
        // chunk's scalars while the first waves form the decay mask.
        if (j + 1 < nchunks) {
            const float dtn = st.rdt[0];
            const TrapIn tin = TRAP ? st.rtp[0] : TrapIn{};
            st.template store<0>(Bs[buf ^ 1], Cs[buf ^ 1], Xs[buf ^ 1]);
            if (j + 2 < nchunks) st.template load<0>(t0 + 2 * kT);
            if (wid == NW - 1)
                chunk_scalars(scal[buf ^ 1], dtn, t0 + kT + (lane & 31) < p.L && lane < kT, bias, A, p.mode, lane,
                              TRAP ? &tin : nullptr);
        }

        // D4, shared: G^T[s][t] = B[s].C[t] for the causal tile pairs (s-tile,
        // t-tile) (0,0), (0,1), (1,1), one per wave (wave tau % NW); lane holds
        // column t, rows s = q*4 .. q*4+3.  M[t][s] = G[t][s] e^{cs_t - cs_s}
        // sigma_s (s <= t) goes to LDS as the A fragments of M X, with K slots
        // q*8+i <-> s = q*4+i (i < 4) and 16+q*4+(i-4) (i >= 4).
#pragma unroll
        for (int tau = 0; tau < 3; ++tau) {
            if (tau % NW != wid) continue;
            const int sT = tau == 2 ? 1 : 0, tT = tau == 0 ? 0 : 1;
            f32x4 G{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NMAX; kk += 32) {
                if (kk >= N) break;
                const u32x4 bf = *reinterpret_cast<const u32x4 *>(&B_[(sT * 16 + c16) * BCP + kk + q * 8]);
                const u32x4 cf = *reinterpret_cast<const u32x4 *>(&C_[(tT * 16 + c16) * BCP + kk + q * 8]);
                G = mfma16(bf, cf, G);
            }
            const float4 cs4 = *reinterpret_cast<const float4 *>(&sc.cs[sT * 16 + q * 4]);
            const float4 sg4 = *reinterpret_cast<const float4 *>(&sc.sig[sT * 16 + q * 4]);
            const float4 gm4 = TRAP ? *reinterpret_cast<const float4 *>(&sc.gam[sT * 16 + q * 4]) : sg4;
            const float csA[4] = {cs4.x, cs4.y, cs4.z, cs4.w}, sgA[4] = {sg4.x, sg4.y, sg4.z, sg4.w};
            const float gmA[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
            const float ct = sc.cs[tT * 16 + c16];
            float m[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool keep = (sT < tT) || (q * 4 + i <= c16);     // s <= t
                const bool diag = (sT == tT) && (q * 4 + i == c16);    // s == t
                m[i] = keep ? G[i] * __expf(ct - csA[i]) * (diag ? gmA[i] : sgA[i]) : 0.0f;
            }
            const uint2 u0 = split_bf16(m[0], m[1]), u1 = split_bf16(m[2], m[3]);
            uint32_t *mh = reinterpret_cast<uint32_t *>(&Ms[tT][0][lane]);
            uint32_t *ml = reinterpret_cast<uint32_t *>(&Ms[tT][1][lane]);
            const int dw = sT * 2;       // K slots 0-3 hold s-tile 0, slots 4-7 s-tile 1
            *reinterpret_cast<uint2 *>(mh + dw) = make_uint2(u0.x, u1.x);
            *reinterpret_cast<uint2 *>(ml + dw) = make_uint2(u0.y, u1.y);
            if (tau == 0) {              // s-tile 1 lies above the diagonal of t-tile 0
                *reinterpret_cast<uint2 *>(mh + 2) = make_uint2(0u, 0u);
                *reinterpret_cast<uint2 *>(ml + 2) = make_uint2(0u, 0u);
            }
        }

        // D5: yacc[tt] = C[t][:] S[:][p] for t in time tile tt, then scaled by e^{cs_t}
        f32x4 yacc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int k = 0; k < NT / 2; ++k) {
            if (k * 32 >= N) break;
            const uint2 s0 = split_bf16(S[2 * k][0], S[2 * k][1]);
            const uint2 s1 = split_bf16(S[2 * k][2], S[2 * k][3]);
            const uint2 s2 = split_bf16(S[2 * k + 1][0], S[2 * k + 1][1]);
            const uint2 s3 = split_bf16(S[2 * k + 1][2], S[2 * k + 1][3]);
            const u32x4 Sh{s0.x, s1.x, s2.x, s3.x}, Sl{s0.y, s1.y, s2.y, s3.y};
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint16_t *cr = C_ + (tt * 16 + c16) * BCP + k * 32 + q * 4;
                const uint2 a0 = *reinterpret_cast<const uint2 *>(cr);
                const uint2 a1 = *reinterpret_cast<const uint2 *>(cr + 16);
                const u32x4 Af{a0.x, a0.y, a1.x, a1.y};
                yacc[tt] = mfma16(Af, Sh, yacc[tt]);
                yacc[tt] = mfma16(Af, Sl, yacc[tt]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const float4 e = *reinterpret_cast<const float4 *>(&sc.ecs[tt * 16 + q * 4]);
            yacc[tt][0] *= e.x; yacc[tt][1] *= e.y; yacc[tt][2] *= e.z; yacc[tt][3] *= e.w;
        }

        __syncthreads();   // the shared M fragments are complete; C is consumed

        uint16_t *Wh = W_IN_C ? Cs[buf] + wid * 2 * kT * WP : Wsep[W_IN_C ? 0 : wid];
        uint16_t *Wl = Wh + kT * WP;
        weighted_x<XP>(X_, p0, sc.w, Wh, Wl, lane);

        // D4: yacc[tt] += M X, X fragments read transposed from the x tile
        {
            const uint2 xa0 = tr_read(X_, XP, q * 4, p0, lane);
            const uint2 xa1 = tr_read(X_, XP, 16 + q * 4, p0, lane);
            const u32x4 Xf{xa0.x, xa0.y, xa1.x, xa1.y};
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                yacc[tt] = mfma16(Ms[tt][0][lane], Xf, yacc[tt]);
                yacc[tt] = mfma16(Ms[tt][1][lane], Xf, yacc[tt]);
            }
        }

        // skip term and store: lane (column c16, rows t = tt*16 + q*4 + i); the
        // row base is uniform, the lane adds a 32-bit byte offset
        float yv[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const uint2 xv = tr_read(X_, XP, tt * 16 + q * 4, p0, lane);
            const float xs[4] = {lo_f(xv.x), hi_f(xv.x), lo_f(xv.y), hi_f(xv.y)};
#pragma unroll
            for (int i = 0; i < 4; ++i) yv[tt][i] = fmaf(Dh, xs[i], yacc[tt][i]);
        }
        // raw buffer stores whose record count ends at the chunk's last valid step: the
        // hardware drops a ragged tail's stores, so every chunk issues the same 8 stores with
        // no branch around them, and the wait for the next chunk's prefetched loads does not
        // take in these stores (loads and stores share one counter, which the compiler can
        // only count on a path with a fixed number of stores)
        {
            const int64_t nv = min((int64_t)kT, te - t0);
            const int rec = (int)((nv - 1) * rowX * 4 + 64);   // lane columns < 16: 64 bytes of the last row
            const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(Yg + t0 * rowX, 0, rec, kBufWord3);
            const uint32_t yl = lane_off(ylane);      // re-read per chunk: 8 offsets not held across the loop
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv[tt][i]), yr,
                                                          (int)(yl + (uint32_t)((tt * 16 + i) * rowX) * 4u), 0, 0);
        }

        // D2+D3
        state_update<NT, BCP>(S, B_, Wh, Wl, sc.end, N, lane);

        __syncthreads();
    }

    if (p.h_final && wk.k == p.nseg - 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt * 16 >= N) break;
            float *dst = p.h_final + ((wk.b * p.H + wk.h) * p.P + p0 + c16) * p.N + nt * 16 + q * 4;
            *reinterpret_cast<float4 *>(dst) = make_float4(S[nt][0], S[nt][1], S[nt][2], S[nt][3]);
        }
    }
}

// Trapezoidal form: the carried previous input enters the state before step 0,
// h0' = h0 + dt_0 (1 - trap_0) x_prev (x) k_prev  (the shifted state of step -1).
__global__ void __launch_bounds__(256)
ssd_trap_h0_kernel(SsdKp p, const uint16_t *x_prev, const uint16_t *k_prev, float *h0p) {
    const int64_t PN = p.P * p.N, tot = p.batch * p.H * PN;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= tot) return;
    const int64_t bh = i / PN, e = i % PN, pp = e / p.N, n = e % p.N;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t o = b * p.L * p.H + h;                  // step 0 of (b, h)
    const float c = p.dt[o] * (1.0f - p.trap[o]);
    const float xv = __uint_as_float(((uint32_t)x_prev[bh * p.P + pp]) << 16);
    const float kv = __uint_as_float(((uint32_t)k_prev[bh * p.N + n]) << 16);
    h0p[i] = fmaf(c * xv, kv, p.h0 ? p.h0[i] : 0.0f);
}

struct Plan {
    int64_t nseg, Ls;
};
// Segments.  The (batch, segment, head) groups run in rounds of kResident
// groups per CU (3 waves per SIMD), and a group walks its segment's chunks in
// order, so the scan takes about rounds x segment length.  The count that
// minimises that product is taken (a larger count must win by 3 %, as every
// segment adds a state round trip); no segment is shorter than kMinSeg steps,
// lengths are a multiple of the chunk.  A count whose groups spill a few past a
// full round would run the whole chain twice.
Plan plan(int64_t batch, int64_t L, int64_t H, int64_t P) {
    const int64_t nw = P / 16;                                        // waves per group
    const int64_t per_round = kCUs * std::max<int64_t>(1, kWavesPerCU / nw);
    const int64_t max_seg = std::max<int64_t>(1, std::min<int64_t>(L / kMinSeg, kMaxSeg));
    Plan best{1, (L + kT - 1) / kT * kT};
    int64_t best_cost = -1;
    for (int64_t ns = 1; ns <= max_seg; ++ns) {
        const int64_t Ls = ((L + ns - 1) / ns + kT - 1) / kT * kT;
        const int64_t nseg = (L + Ls - 1) / Ls;
        const int64_t rounds = (batch * H * nseg + per_round - 1) / per_round;
        const int64_t cost = rounds * Ls;
        if (best_cost < 0 || cost * 100 < best_cost * 97) {
            best = Plan{nseg, Ls};
            best_cost = cost;
        }
    }
    return best;
}
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

template <int NMAX, bool EXACT, int NW, bool TRAP>
void launch_all(const SsdKp &p, hipStream_t stream) {
    if (p.nseg > 1) {
        // two heads per work group where a group's head count is even, B's
        // pieces divide over the doubled thread count and the pairs fill at
        // least one round of the chip (two per CU): below that, half as many
        // work groups of twice the size load the CUs less evenly
        constexpr bool PAIR_OK = !TRAP && NW <= 4 && (kT * (NMAX / 8)) % (128 * NW) == 0;
        if (PAIR_OK && (p.H / p.G) % 2 == 0 && p.batch * (p.nseg - 1) * (p.H / 2) >= 2 * kCUs) {
            const int64_t n1 = p.batch * (p.nseg - 1) * (p.H / 2);
            hipLaunchKernelGGL((ssd_state_kernel<NMAX, EXACT, NW, TRAP, PAIR_OK ? 2 : 1>), dim3((unsigned)n1),
                               dim3(128 * NW), 0, stream, p);
        } else {
            const int64_t n1 = p.batch * (p.nseg - 1) * p.H;
            hipLaunchKernelGGL((ssd_state_kernel<NMAX, EXACT, NW, TRAP, 1>), dim3((unsigned)n1), dim3(64 * NW), 0,
                               stream, p);
        }
        const int64_t nt = p.batch * p.H * p.P * p.N / 4;
        hipLaunchKernelGGL(ssd_pass_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, stream, p);
    }
    const int64_t n = p.batch * p.nseg * p.H;
    hipLaunchKernelGGL((ssd_scan_kernel<NMAX, EXACT, NW, TRAP>), dim3((unsigned)n), dim3(64 * NW), 0, stream, p);
}

template <int NW, bool TRAP>
void launch_n(const SsdKp &p, hipStream_t stream) {
    // the B/C tile is at least P wide so that its pieces divide over the group
    constexpr int NMIN = 16 * NW < 64 ? 64 : 16 * NW;
    if constexpr (NMIN == 64) {
        if (p.N == 64) return launch_all<64, true, NW, TRAP>(p, stream);
        if (p.N < 64) return launch_all<64, false, NW, TRAP>(p, stream);
    }
    if (p.N == 128) return launch_all<128, true, NW, TRAP>(p, stream);
    if (p.N < 128) return launch_all<128, false, NW, TRAP>(p, stream);
    if (p.N == 256) return launch_all<256, true, NW, TRAP>(p, stream);
    launch_all<256, false, NW, TRAP>(p, stream);
}

}  // namespace

size_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                           int64_t) {
    const Plan pl = plan(batch, L, nheads, headdim);
    if (pl.nseg <= 1) return 0;
    return align256((size_t)(batch * nheads * pl.nseg * headdim * d_state) * sizeof(float)) +
           (size_t)(batch * nheads * pl.nseg) * sizeof(float);
}

size_t ssd_trap_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state) {
    return align256(ssd_workspace_bytes(batch, L, nheads, headdim, d_state, 0)) +
           align256((size_t)(batch * nheads * headdim * d_state) * sizeof(float));
}

hipError_t launch_ssd_trap(const SsdTrapArgs &a, hipStream_t stream, const char **kernel_name) {
    if (a.L == 1) return launch_ssd_trap_step(a, stream, kernel_name);   // a decode step
    *kernel_name = "ssd_scan_kernel";
    SsdKp p{};
    p.x = static_cast<const uint16_t *>(a.x);
    p.dt = a.dt; p.dt_bias = nullptr; p.A_log = nullptr;
    p.B = static_cast<const uint16_t *>(a.k);
    p.C = static_cast<const uint16_t *>(a.q);
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.H = a.nheads; p.P = a.headdim; p.N = a.d_state; p.G = a.nheads;
    p.mode = 1;
    p.aval = a.a; p.trap = a.trap;
    const Plan pl = plan(p.batch, p.L, p.H, p.P);
    p.nseg = pl.nseg;
    p.Ls = pl.Ls;
    char *ws = static_cast<char *>(a.workspace);
    if (p.nseg > 1) {
        p.ws_state = reinterpret_cast<float *>(ws);
        p.ws_decay = reinterpret_cast<float *>(ws + align256((size_t)(p.batch * p.H * p.nseg * p.P * p.N) * sizeof(float)));
    }
    if (a.x_prev) {
        float *h0p = reinterpret_cast<float *>(ws + align256(ssd_workspace_bytes(p.batch, p.L, p.H, p.P, p.N, 0)));
        const int64_t tot = p.batch * p.H * p.P * p.N;
        *kernel_name = "ssd_trap_h0_kernel";
        hipLaunchKernelGGL(ssd_trap_h0_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, p,
                           static_cast<const uint16_t *>(a.x_prev), static_cast<const uint16_t *>(a.k_prev), h0p);
        p.h0 = h0p;
        *kernel_name = "ssd_scan_kernel";
    }
    if (p.P == 32) launch_n<2, true>(p, stream);
    else if (p.P == 64) launch_n<4, true>(p, stream);
    else launch_n<8, true>(p, stream);
    return hipGetLastError();
}

hipError_t launch_ssd_trap_h0(const void *x_prev, const void *k_prev, const float *dt, const float *trap,
                              const float *h0, float *h0p, int64_t batch, int64_t L, int64_t nheads,
                              int64_t headdim, int64_t d_state, hipStream_t stream) {
    SsdKp p{};
    p.dt = dt; p.trap = trap; p.h0 = h0;
    p.batch = batch; p.L = L; p.H = nheads; p.P = headdim; p.N = d_state;
    const int64_t tot = batch * nheads * headdim * d_state;
    hipLaunchKernelGGL(ssd_trap_h0_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, p,
                       static_cast<const uint16_t *>(x_prev), static_cast<const uint16_t *>(k_prev), h0p);
    return hipGetLastError();
}

hipError_t launch_ssd(const SsdArgs &a, hipStream_t stream, const char **kernel_name) {
    if (a.L == 1) return launch_ssd_step(a, stream, kernel_name);   // a decode step (ssd_decode.hip)
    *kernel_name = "ssd_scan_kernel";
    SsdKp p{};
    p.x = static_cast<const uint16_t *>(a.x);
    p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log;
    p.B = static_cast<const uint16_t *>(a.B);
    p.C = static_cast<const uint16_t *>(a.C);
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.H = a.nheads; p.P = a.headdim; p.N = a.d_state; p.G = a.ngroups;
    p.mode = (int)(a.flags & 0x3u);
    const Plan pl = plan(p.batch, p.L, p.H, p.P);
    p.nseg = pl.nseg;
    p.Ls = pl.Ls;
    if (p.nseg > 1) {
        p.ws_state = static_cast<float *>(a.workspace);
        p.ws_decay = reinterpret_cast<float *>(
            static_cast<char *>(a.workspace) +
            align256((size_t)(p.batch * p.H * p.nseg * p.P * p.N) * sizeof(float)));
    }
    if (p.P == 32) launch_n<2, false>(p, stream);
    else if (p.P == 64) launch_n<4, false>(p, stream);
    else launch_n<8, false>(p, stream);
    return hipGetLastError();
}

}  // namespace ssm
