// cssd_scan.hip -- complex-state SSD (Mamba-3 SISO style) chunked forward scan.
//
// Follows builderforce-memory-engine complex_ssd.ts (header comment,
// et_bbar_re/et_bbar_im, complex_ssd_forward): a complex diagonal state per
// (head channel p, complex state n), complex decay Abar_t = exp(delta_t*mu),
// complex input scale beta_t, output Re(C.h) + D x.  With a head-constant mu the
// decay from step s to step t is exp(mu * (Lambda_t - Lambda_s)), Lambda the
// running sum of delta, so the same chunked decomposition as the real SSD
// applies:
//   K1  Shat_c[p,n] = sum_s exp(mu(Lambda_end - Lambda_s)) beta_s B_s[n] x_s[p]
//   K2  S_{c+1} = exp(mu Lambda_end(c)) S_c + Shat_c,  h_final = S_nc
//   K3  y_t[p] = sum_{s<=t} Re(G[t,s] exp(mu(Lambda_t-Lambda_s)) beta_s) x_s[p]
//              + Re(sum_n C_t[n] exp(mu Lambda_t) S_c[p,n]) + D x_t[p],
//       G[t,s] = sum_n C_t[n] B_s[n]
// Every decay factor is taken between two steps of one chunk (or from the chunk
// start), so for the stable reading of A no exponent is positive.
// Arithmetic is fp32 on the vector ALUs.
#include "device_common.hpp"
#include "launchers.hpp"

namespace ssm {
namespace {

constexpr int kThreads = 256;

struct CssdKp {
    const float *x; const float *dt; const float *dt_bias; const float *A_log;
    const float *B; const float *C; const float *D; float *y;
    const float *h0; float *h_final;
    float *states;      // [batch][nc][H][P][Nc][2]
    float *cdec;        // [batch][H][nc][2]   exp(mu * Lambda_end) per chunk
    int64_t batch, L, H, P, Nc, G, nc;
    uint32_t flags;
};

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

// mu (the per-unit-delta complex rate) of head h for the selected reading
__device__ __forceinline__ cf head_mu(const CssdKp &p, int64_t h) {
    const float ell = p.A_log[2 * h], phi = p.A_log[2 * h + 1];
    const uint32_t am = p.flags & 0xCu;
    if (am == 0x4u) { float s, c; sincosf(phi, &s, &c); const float m = expf(ell); return {m * c, m * s}; }
    if (am == 0x8u) return {ell, phi};
    return {-expf(ell), phi};
}

__device__ __forceinline__ cf input_scale(const CssdKp &p, int64_t h, cf mu, float dl) {
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

// per-chunk scalars: Lam[t] = inclusive running sum of delta (0 past L),
// bet[t] = beta_t (0 past L).  The rotation angle phi*(Lam_t - Lam_s) turns an
// absolute error of Lam into a relative error of the output, so delta and its
// running sum are formed in double precision (Q values per chunk); every
// difference of two Lam is taken in double and only then rounded to fp32.
template <int Q>
__device__ __forceinline__ void chunk_scalars(const CssdKp &p, int64_t b, int64_t c, int64_t h, cf mu,
                                              double *Lam, float *bre, float *bim, double *wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const double bias = p.dt_bias ? (double)p.dt_bias[h] : 0.0;
    double dl = 0.0;
    cf be{0.0f, 0.0f};
    const int64_t t = c * Q + tid;
    if (tid < Q && t < p.L) {
        const double xv = (double)p.dt[(b * p.L + t) * p.H + h] + bias;
        dl = xv > 0.0 ? xv + log1p(exp(-xv)) : log1p(exp(xv));   // softplus
        be = input_scale(p, h, mu, (float)dl);
    }
    double v = dl;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    if (lane == 63) wsum[wid] = v;
    __syncthreads();
    double pre = 0.0;
    for (int w = 0; w < wid; ++w) pre += wsum[w];
    if (tid < Q) { Lam[tid] = v + pre; bre[tid] = be.re; bim[tid] = be.im; }
    __syncthreads();
}

template <int Q>
__global__ void __launch_bounds__(kThreads)
cssd_chunk_state_kernel(CssdKp p) {
    __shared__ double Lam[Q], wsum[4];
    __shared__ float bre[Q], bim[Q], wre[Q], wim[Q];
    const int64_t work = xcd_swizzle(blockIdx.x, p.batch * p.nc * p.H);
    const int64_t h = work % p.H, c = (work / p.H) % p.nc, b = work / (p.H * p.nc);
    const int64_t g = h * p.G / p.H;
    const int tid = threadIdx.x;
    const cf mu = head_mu(p, h);
    chunk_scalars<Q>(p, b, c, h, mu, Lam, bre, bim, wsum);
    const double Lend = Lam[Q - 1];
    if (tid < Q) {   // w_s = exp(mu (Lambda_end - Lambda_s)) beta_s
        const float dlam = (float)(Lend - Lam[tid]);
        const cf e = cexpf_(mu.re * dlam, mu.im * dlam);
        const cf w = cmul(e, cf{bre[tid], bim[tid]});
        wre[tid] = w.re; wim[tid] = w.im;
    }
    if (tid == 0) {
        const cf e = cexpf_(mu.re * (float)Lend, mu.im * (float)Lend);
        p.cdec[((b * p.H + h) * p.nc + c) * 2] = e.re;
        p.cdec[((b * p.H + h) * p.nc + c) * 2 + 1] = e.im;
    }
    __syncthreads();
    const int64_t smax = min((int64_t)Q, p.L - c * Q);
    for (int64_t e = tid; e < p.P * p.Nc; e += kThreads) {
        const int64_t pp = e / p.Nc, n = e % p.Nc;
        // four interleaved partial sums: shorter fp32 rounding chains
        float are[4] = {0.0f, 0.0f, 0.0f, 0.0f}, aim[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int64_t s = 0; s < smax; ++s) {
            const int64_t t = c * Q + s;
            const float xv = p.x[((b * p.L + t) * p.H + h) * p.P + pp];
            const float *Bs = p.B + (((b * p.L + t) * p.G + g) * p.Nc + n) * 2;
            const cf wb = cmul(cf{wre[s], wim[s]}, cf{Bs[0], Bs[1]});
            are[s & 3] = fmaf(wb.re, xv, are[s & 3]);
            aim[s & 3] = fmaf(wb.im, xv, aim[s & 3]);
        }
        float *dst = p.states + ((((b * p.nc + c) * p.H + h) * p.P + pp) * p.Nc + n) * 2;
        dst[0] = (are[0] + are[1]) + (are[2] + are[3]);
        dst[1] = (aim[0] + aim[1]) + (aim[2] + aim[3]);
    }
}

__global__ void __launch_bounds__(kThreads)
cssd_state_pass_kernel(CssdKp p) {
    const int64_t PN = p.P * p.Nc;
    const int64_t per_bh = (PN + kThreads - 1) / kThreads;
    const int64_t bh = blockIdx.x / per_bh;
    const int64_t e = (blockIdx.x % per_bh) * kThreads + threadIdx.x;
    if (e >= PN) return;
    const int64_t b = bh / p.H, h = bh % p.H;
    cf S{0.0f, 0.0f};
    if (p.h0) { S.re = p.h0[(bh * PN + e) * 2]; S.im = p.h0[(bh * PN + e) * 2 + 1]; }
    for (int64_t c = 0; c < p.nc; ++c) {
        float *st = p.states + (((b * p.nc + c) * p.H + h) * PN + e) * 2;
        const cf loc{st[0], st[1]};
        st[0] = S.re; st[1] = S.im;
        const float *d = p.cdec + ((b * p.H + h) * p.nc + c) * 2;
        const cf dec{d[0], d[1]};
        const cf n = cmul(dec, S);
        S = {n.re + loc.re, n.im + loc.im};
    }
    if (p.h_final) { p.h_final[(bh * PN + e) * 2] = S.re; p.h_final[(bh * PN + e) * 2 + 1] = S.im; }
}

template <int Q>
__global__ void __launch_bounds__(kThreads)
cssd_chunk_scan_kernel(CssdKp p) {
    __shared__ double Lam[Q], wsum[4];
    __shared__ float bre[Q], bim[Q], e0re[Q], e0im[Q];
    __shared__ float M[Q][Q + 1];
    const int64_t work = xcd_swizzle(blockIdx.x, p.batch * p.nc * p.H);
    const int64_t h = work % p.H, c = (work / p.H) % p.nc, b = work / (p.H * p.nc);
    const int64_t g = h * p.G / p.H;
    const int tid = threadIdx.x;
    const cf mu = head_mu(p, h);
    const float csign = (p.flags & 0x10u) ? -1.0f : 1.0f;   // conj(C)
    chunk_scalars<Q>(p, b, c, h, mu, Lam, bre, bim, wsum);
    if (tid < Q) {
        const float lt = (float)Lam[tid];
        const cf e = cexpf_(mu.re * lt, mu.im * lt);
        e0re[tid] = e.re; e0im[tid] = e.im;
    }
    const int64_t tmax = min((int64_t)Q, p.L - c * Q);
    // M[t][s] = Re(G[t,s] exp(mu(Lambda_t - Lambda_s)) beta_s), s <= t
    for (int e = tid; e < Q * Q; e += kThreads) {
        const int t = e / Q, s = e % Q;
        float m = 0.0f;
        if (s <= t && t < tmax) {
            const float *Ct = p.C + ((b * p.L + c * Q + t) * p.G + g) * p.Nc * 2;
            const float *Bs = p.B + ((b * p.L + c * Q + s) * p.G + g) * p.Nc * 2;
            float gre2[2] = {0.0f, 0.0f}, gim2[2] = {0.0f, 0.0f};
            for (int64_t n = 0; n < p.Nc; ++n) {
                const float cr = Ct[2 * n], ci = csign * Ct[2 * n + 1];
                const float br = Bs[2 * n], bi = Bs[2 * n + 1];
                gre2[n & 1] = fmaf(cr, br, fmaf(-ci, bi, gre2[n & 1]));
                gim2[n & 1] = fmaf(cr, bi, fmaf(ci, br, gim2[n & 1]));
            }
            const float gre = gre2[0] + gre2[1], gim = gim2[0] + gim2[1];
            const float dlam = (float)(Lam[t] - Lam[s]);
            const cf ex = cexpf_(mu.re * dlam, mu.im * dlam);
            const cf k = cmul(cmul(cf{gre, gim}, ex), cf{bre[s], bim[s]});
            m = k.re;
        }
        M[t][s] = m;
    }
    __syncthreads();
    const float Dh = p.D ? p.D[h] : 0.0f;
    const bool has_state = (c > 0) || (p.h0 != nullptr);
    const float *Sb = p.states + ((b * p.nc + c) * p.H + h) * p.P * p.Nc * 2;
    for (int64_t e = tid; e < tmax * p.P; e += kThreads) {
        const int64_t t = e / p.P, pp = e % p.P;
        float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int64_t s = 0; s <= t; ++s)
            a4[s & 3] = fmaf(M[t][s], p.x[((b * p.L + c * Q + s) * p.H + h) * p.P + pp], a4[s & 3]);
        float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
        if (has_state) {
            const float *Ct = p.C + ((b * p.L + c * Q + t) * p.G + g) * p.Nc * 2;
            const float *Sp = Sb + pp * p.Nc * 2;
            const cf e0{e0re[t], e0im[t]};
            float s2[2] = {0.0f, 0.0f};
            for (int64_t n = 0; n < p.Nc; ++n) {
                const cf cc = cmul(cf{Ct[2 * n], csign * Ct[2 * n + 1]}, e0);
                s2[n & 1] = fmaf(cc.re, Sp[2 * n], fmaf(-cc.im, Sp[2 * n + 1], s2[n & 1]));
            }
            acc += s2[0] + s2[1];
        }
        const float xv = p.x[((b * p.L + c * Q + t) * p.H + h) * p.P + pp];
        p.y[((b * p.L + c * Q + t) * p.H + h) * p.P + pp] = fmaf(Dh, xv, acc);
    }
}

template <int Q>
hipError_t launch_q(const CssdKp &kp, hipStream_t s) {
    const int64_t nwork = kp.batch * kp.nc * kp.H;
    hipLaunchKernelGGL((cssd_chunk_state_kernel<Q>), dim3((unsigned)nwork), dim3(kThreads), 0, s, kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t per_bh = (kp.P * kp.Nc + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(cssd_state_pass_kernel, dim3((unsigned)(kp.batch * kp.H * per_bh)), dim3(kThreads), 0, s, kp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((cssd_chunk_scan_kernel<Q>), dim3((unsigned)nwork), dim3(kThreads), 0, s, kp);
    return hipGetLastError();
}

}  // namespace

size_t cssd_workspace_bytes(int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                            int64_t n_complex, int64_t chunk_len) {
    const int64_t nc = (L + chunk_len - 1) / chunk_len;
    const size_t st = (size_t)batch * nc * nheads * headdim * n_complex * 2 * sizeof(float);
    const size_t cd = (size_t)batch * nheads * nc * 2 * sizeof(float);
    return ((st + 255) / 256) * 256 + ((cd + 255) / 256) * 256;
}

hipError_t launch_cssd(const CssdArgs &a, hipStream_t stream, const char **kernel_name) {
    *kernel_name = "cssd_chunk_state_kernel/cssd_state_pass_kernel/cssd_chunk_scan_kernel";
    CssdKp p{};
    p.x = a.x; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C;
    p.D = a.D; p.y = a.y; p.h0 = a.h0; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.H = a.nheads; p.P = a.headdim; p.Nc = a.n_complex; p.G = a.ngroups;
    p.nc = (a.L + a.chunk_len - 1) / a.chunk_len;
    const size_t st = (size_t)a.batch * p.nc * a.nheads * a.headdim * a.n_complex * 2 * sizeof(float);
    p.states = static_cast<float *>(a.workspace);
    p.cdec = reinterpret_cast<float *>(static_cast<char *>(a.workspace) + ((st + 255) / 256) * 256);
    p.flags = a.flags;
    if (a.chunk_len == 32) return launch_q<32>(p, stream);
    if (a.chunk_len == 64) return launch_q<64>(p, stream);
    return launch_q<128>(p, stream);
}

}  // namespace ssm
