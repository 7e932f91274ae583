/*
 * ssm_oracle.c -- plain, slow, fp64 CPU oracle for the forward selective
 * state-space scans.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests,
 * by the package smoke check and by the CPU-baseline leg of the benchmark,
 * never by the product path.  It shares no source, header, table or helper
 * with the HIP library.
 *
 * Every function runs the sequential recurrence exactly as the pages define
 * it, one independent unit at a time, in double precision:
 *
 *   S6 (per batch b, channel d, state n) -- builderforce-memory-engine
 *   2026.6.18, dist/kernels/selective_scan.js, header comment and the
 *   helpers softplus / discretise_A / discretise_B:
 *       delta_t = softplus(dt[b,t,d] + dt_bias[d])
 *       A       = -exp(A_log[d,n])
 *       Abar    = exp(delta_t * A)
 *       beta    = (Abar - 1)/A            (zero-order hold; = delta*phi1(delta*A))
 *       h_t     = Abar*h_{t-1} + beta*B[b,t,n]*u[b,t,d]
 *       y[b,t,d]= sum_n C[b,t,n]*h_t[n] + D[d]*u[b,t,d]
 *
 *   SSD (per batch b, head h, channel p, state n) -- same package,
 *   dist/kernels/ssd.js, header comment and ssd_chunk_forward, read with
 *   A = -exp(A_log[h]) and an input scale sigma_t (delta_t by default):
 *       a_t     = delta_t * A_h
 *       S_t     = exp(a_t)*S_{t-1} + sigma_t * x[b,t,h,p] * B[b,t,g,n]
 *       y[b,t,h,p] = sum_n C[b,t,g,n]*S_t[p,n] + D[h]*x[b,t,h,p]
 *     with group g = floor(h*G/H).
 *
 *   Complex SSD -- same package, src/kernels/complex_ssd.ts, header comment
 *   and complex_ssd_forward: complex state per (p, n_c), complex decay
 *   Abar = exp(delta*lambda_h), exponential-trapezoid input scale
 *   beta = (Abar - 1)/lambda_h, output Re(C.h) + D x.
 *
 * The chunked decomposition the GPU uses is NOT here: the oracle is the
 * definition, and the tests check the chunked algebra against it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

/* flag values of the library interface, restated here by value */
#define OR_BBAR_MASK   0x3
#define OR_BBAR_ZOH    0x0
#define OR_BBAR_DT     0x1
#define OR_BBAR_ONE    0x2
#define OR_CPLX_MASK   0xC
#define OR_CPLX_STABLE 0x0
#define OR_CPLX_DOC    0x4
#define OR_CPLX_CODE   0x8
#define OR_CPLX_CONJ_C 0x10

/* softplus(x) = log(1 + e^x), evaluated without overflow.  The pages write
 * it as log(1 + exp(x)) (selective_scan.js and ssd.js, fn softplus); this
 * is the same function. */
static double sp(double x)
{
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/* phi1(z) = (e^z - 1)/z, phi1(0) = 1: the zero-order-hold factor, so that
 * (exp(delta*A) - 1)/A = delta * phi1(delta*A) also at A = 0. */
static double phi1(double z)
{
    return z == 0.0 ? 1.0 : expm1(z) / z;
}

/* ---------------------------------------------------------------- S6 --- */

typedef struct {
    const float *u, *dt, *dt_bias, *A_log, *B, *C, *D, *h0;
    int64_t batch, L, Dm, N;
    uint32_t flags;
    const int64_t *units;   /* pairs (b, d) */
    int64_t n_units;
    double *y_out;          /* [n_units][L] */
    double *hf_out;         /* [n_units][N] or NULL */
    /* layer form (oracle_s6_layer_fwd): u from a causal conv of x, gated output */
    const float *conv_w, *conv_b, *conv_state, *z;   /* conv_w NULL: plain scan of u */
    int64_t K;
    double *u_out;          /* [n_units][L] or NULL */
    double *cs_out;         /* [n_units][K-1] or NULL */
    /* grouped B, C (oracle_s6_grouped_fwd): (batch, L, G, N), channel d reads
     * group d*G/Dm (G = Dm: per channel); 0 means one shared (batch, L, N) */
    int64_t G;
} s6_job;

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* x of unit (b, d) at time t, extended to t < 0 by the carried conv state
 * (conv_state[b, d, K-1+t], oldest first) or zeros */
static double conv_x(const s6_job *j, int64_t b, int64_t d, int64_t t)
{
    if (t >= 0) return (double)j->u[(b * j->L + t) * j->Dm + d];
    if (!j->conv_state) return 0.0;
    return (double)j->conv_state[(b * j->Dm + d) * (j->K - 1) + (j->K - 1) + t];
}

static void s6_unit(const s6_job *j, int64_t k)
{
    const int64_t b = j->units[2 * k], d = j->units[2 * k + 1];
    const int64_t L = j->L, Dm = j->Dm, N = j->N;
    const int mode = (int)(j->flags & OR_BBAR_MASK);
    double *A = (double *)malloc(sizeof(double) * (size_t)N);
    double *h = (double *)malloc(sizeof(double) * (size_t)N);
    for (int64_t n = 0; n < N; ++n) {
        A[n] = -exp((double)j->A_log[d * N + n]);
        h[n] = j->h0 ? (double)j->h0[(b * Dm + d) * N + n] : 0.0;
    }
    const double bias = j->dt_bias ? (double)j->dt_bias[d] : 0.0;
    const double Dd = j->D ? (double)j->D[d] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t e = (b * L + t) * Dm + d;
        const double delta = sp((double)j->dt[e] + bias);
        double uu;
        if (j->conv_w) {      /* u_t = SiLU(sum_k w[d,k] x_{t-k} + bias[d]) */
            double pre = j->conv_b ? (double)j->conv_b[d] : 0.0;
            for (int64_t q = 0; q < j->K; ++q) pre += (double)j->conv_w[d * j->K + q] * conv_x(j, b, d, t - q);
            uu = silu(pre);
            if (j->u_out) j->u_out[k * L + t] = uu;
        } else {
            uu = (double)j->u[e];
        }
        const int64_t G = j->G > 0 ? j->G : 1, g = d * G / Dm;
        const float *Bt = j->B + ((b * L + t) * G + g) * N;
        const float *Ct = j->C + ((b * L + t) * G + g) * N;
        double yv = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double z = delta * A[n];
            double beta;
            if (mode == OR_BBAR_ZOH) beta = delta * phi1(z);
            else if (mode == OR_BBAR_DT) beta = delta;
            else beta = 1.0;
            h[n] = exp(z) * h[n] + beta * (double)Bt[n] * uu;
            yv += (double)Ct[n] * h[n];
        }
        const double yt = yv + Dd * uu;
        j->y_out[k * L + t] = (j->conv_w && j->z) ? yt * silu((double)j->z[e]) : yt;
    }
    if (j->hf_out)
        for (int64_t n = 0; n < N; ++n) j->hf_out[k * N + n] = h[n];
    if (j->conv_w && j->cs_out)
        for (int64_t q = 0; q < j->K - 1; ++q) j->cs_out[k * (j->K - 1) + q] = conv_x(j, b, d, L - (j->K - 1) + q);
    free(A);
    free(h);
}

/* ---------------------------------------------------------------- SSD --- */

typedef struct {
    const float *x, *dt, *dt_bias, *A_log, *B, *C, *D, *h0;
    int64_t batch, L, H, P, N, G;
    uint32_t flags;
    const int64_t *units;   /* pairs (b, h) */
    int64_t n_units;
    double *y_out;          /* [n_units][L][P] */
    double *hf_out;         /* [n_units][P][N] or NULL */
} ssd_job;

static void ssd_unit(const ssd_job *j, int64_t k)
{
    const int64_t b = j->units[2 * k], hh = j->units[2 * k + 1];
    const int64_t L = j->L, H = j->H, P = j->P, N = j->N, G = j->G;
    const int64_t g = hh * G / H;
    const int mode = (int)(j->flags & OR_BBAR_MASK);
    const double A = -exp((double)j->A_log[hh]);
    const double bias = j->dt_bias ? (double)j->dt_bias[hh] : 0.0;
    const double Dh = j->D ? (double)j->D[hh] : 0.0;
    double *S = (double *)malloc(sizeof(double) * (size_t)(P * N));
    for (int64_t i = 0; i < P * N; ++i)
        S[i] = j->h0 ? (double)j->h0[(b * H + hh) * P * N + i] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const double delta = sp((double)j->dt[(b * L + t) * H + hh] + bias);
        const double a = delta * A;
        double sigma;
        if (mode == OR_BBAR_DT) sigma = delta;
        else if (mode == OR_BBAR_ZOH) sigma = delta * phi1(a);
        else sigma = 1.0;
        const double dec = exp(a);
        const float *xt = j->x + ((b * L + t) * H + hh) * P;
        const float *Bt = j->B + ((b * L + t) * G + g) * N;
        const float *Ct = j->C + ((b * L + t) * G + g) * N;
        double *yt = j->y_out + (k * L + t) * P;
        for (int64_t p = 0; p < P; ++p) {
            const double xv = (double)xt[p];
            double *Sp = S + p * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                Sp[n] = dec * Sp[n] + sigma * xv * (double)Bt[n];
                acc += (double)Ct[n] * Sp[n];
            }
            yt[p] = acc + Dh * xv;
        }
    }
    if (j->hf_out) memcpy(j->hf_out + k * P * N, S, sizeof(double) * (size_t)(P * N));
    free(S);
}

/* ------------------------------------------------------- complex SSD --- */

typedef struct { double re, im; } cplx;

static cplx cmul(cplx a, cplx b) { cplx r = {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; return r; }
static cplx cdivc(cplx a, cplx b)
{
    const double den = b.re * b.re + b.im * b.im;
    cplx r = {(a.re * b.re + a.im * b.im) / den, (a.im * b.re - a.re * b.im) / den};
    return r;
}
static cplx cexp_(cplx w) { const double m = exp(w.re); cplx r = {m * cos(w.im), m * sin(w.im)}; return r; }
/* e^w - 1 without cancellation: Re = expm1(x)cos(y) - 2 sin^2(y/2), Im = e^x sin(y) */
static cplx cexpm1_(cplx w)
{
    const double s = sin(0.5 * w.im);
    cplx r = {expm1(w.re) * cos(w.im) - 2.0 * s * s, exp(w.re) * sin(w.im)};
    return r;
}
/* complex phi1(w) = (e^w - 1)/w, phi1(0) = 1 */
static cplx cphi1(cplx w)
{
    if (w.re == 0.0 && w.im == 0.0) { cplx one = {1.0, 0.0}; return one; }
    return cdivc(cexpm1_(w), w);
}

typedef struct {
    const float *x, *dt, *dt_bias, *A_log, *B, *C, *D, *h0;
    int64_t batch, L, H, P, Nc, G;
    uint32_t flags;
    const int64_t *units;
    int64_t n_units;
    double *y_out;          /* [n_units][L][P] */
    double *hf_out;         /* [n_units][P][Nc][2] or NULL */
} cssd_job;

static void cssd_unit(const cssd_job *j, int64_t k)
{
    const int64_t b = j->units[2 * k], hh = j->units[2 * k + 1];
    const int64_t L = j->L, H = j->H, P = j->P, Nc = j->Nc, G = j->G;
    const int64_t g = hh * G / H;
    const int bmode = (int)(j->flags & OR_BBAR_MASK);
    const int amode = (int)(j->flags & OR_CPLX_MASK);
    const int conj_c = (j->flags & OR_CPLX_CONJ_C) != 0;
    const double ell = (double)j->A_log[2 * hh], phi = (double)j->A_log[2 * hh + 1];
    const double bias = j->dt_bias ? (double)j->dt_bias[hh] : 0.0;
    const double Dh = j->D ? (double)j->D[hh] : 0.0;
    cplx lam;
    if (amode == OR_CPLX_DOC) { lam.re = exp(ell) * cos(phi); lam.im = exp(ell) * sin(phi); }
    else { lam.re = -exp(ell); lam.im = phi; }      /* stable reading */
    cplx *S = (cplx *)malloc(sizeof(cplx) * (size_t)(P * Nc));
    for (int64_t i = 0; i < P * Nc; ++i) {
        if (j->h0) {
            S[i].re = (double)j->h0[((b * H + hh) * P * Nc + i) * 2];
            S[i].im = (double)j->h0[((b * H + hh) * P * Nc + i) * 2 + 1];
        } else { S[i].re = 0.0; S[i].im = 0.0; }
    }
    for (int64_t t = 0; t < L; ++t) {
        const double delta = sp((double)j->dt[(b * L + t) * H + hh] + bias);
        cplx abar, beta;
        if (amode == OR_CPLX_CODE) {
            /* the page kernel taken literally: Abar = exp(delta*log|A| + i*delta*arg A),
             * beta = (Abar - 1) * exp(-log|A| - i*arg A) */
            cplx w = {delta * ell, delta * phi};
            cplx inv = {-ell, -phi};
            abar = cexp_(w);
            beta = cmul(cexpm1_(w), cexp_(inv));
        } else {
            cplx w = {delta * lam.re, delta * lam.im};
            abar = cexp_(w);
            if (bmode == OR_BBAR_ZOH) { cplx f = cphi1(w); beta.re = delta * f.re; beta.im = delta * f.im; }
            else if (bmode == OR_BBAR_DT) { beta.re = delta; beta.im = 0.0; }
            else { beta.re = 1.0; beta.im = 0.0; }
        }
        const float *xt = j->x + ((b * L + t) * H + hh) * P;
        const float *Bt = j->B + ((b * L + t) * G + g) * Nc * 2;
        const float *Ct = j->C + ((b * L + t) * G + g) * Nc * 2;
        double *yt = j->y_out + (k * L + t) * P;
        for (int64_t p = 0; p < P; ++p) {
            const double xv = (double)xt[p];
            cplx *Sp = S + p * Nc;
            double acc = 0.0;
            for (int64_t n = 0; n < Nc; ++n) {
                cplx Bn = {(double)Bt[2 * n], (double)Bt[2 * n + 1]};
                cplx inp = cmul(beta, Bn);
                cplx hn = cmul(abar, Sp[n]);
                hn.re += inp.re * xv;
                hn.im += inp.im * xv;
                Sp[n] = hn;
                const double cr = (double)Ct[2 * n], ci = (double)Ct[2 * n + 1];
                acc += conj_c ? (cr * hn.re + ci * hn.im) : (cr * hn.re - ci * hn.im);
            }
            yt[p] = acc + Dh * xv;
        }
    }
    if (j->hf_out)
        for (int64_t i = 0; i < P * Nc; ++i) {
            j->hf_out[(k * P * Nc + i) * 2] = S[i].re;
            j->hf_out[(k * P * Nc + i) * 2 + 1] = S[i].im;
        }
    free(S);
}

/* ------------------------------------------------- complex MIMO SSD --- */
/*
 * The multi-input multi-output form of the complex SSD (builderforce-memory-
 * engine mamba3_block.ts, module header item 2 and the in_proj widths: each
 * head takes R input vectors x^r_t and gives R outputs y^r_t, with B^r_t, C^r_t
 * of Nc complex entries per rank index r).  Per (b, head), with the decay and
 * the input scale of the complex SSD above:
 *   S_t   = Abar_t S_{t-1} + beta_t sum_r (B^r_t x^r_t^T)
 *   y^r_t = Re(C^r_t . S_t) + D x^r_t
 * All R inputs of step t enter S_t before any output of step t is read.
 * Layouts: x, y (batch, L, R, H, P); B, C (batch, L, R, G, Nc, 2); dt (batch, L, H).
 */
typedef struct {
    const float *x, *dt, *dt_bias, *A_log, *B, *C, *D, *h0;
    int64_t batch, L, R, H, P, Nc, G;
    uint32_t flags;
    const int64_t *units;
    int64_t n_units;
    double *y_out;          /* [n_units][L][R][P] */
    double *hf_out;         /* [n_units][P][Nc][2] or NULL */
} mimo_job;

static void mimo_unit(const mimo_job *j, int64_t k)
{
    const int64_t b = j->units[2 * k], hh = j->units[2 * k + 1];
    const int64_t L = j->L, R = j->R, H = j->H, P = j->P, Nc = j->Nc, G = j->G;
    const int64_t g = hh * G / H;
    const int bmode = (int)(j->flags & OR_BBAR_MASK);
    const int conj_c = (j->flags & OR_CPLX_CONJ_C) != 0;
    const double ell = (double)j->A_log[2 * hh], phi = (double)j->A_log[2 * hh + 1];
    const double bias = j->dt_bias ? (double)j->dt_bias[hh] : 0.0;
    const double Dh = j->D ? (double)j->D[hh] : 0.0;
    const cplx lam = {-exp(ell), phi};               /* the stable reading of A */
    cplx *S = (cplx *)malloc(sizeof(cplx) * (size_t)(P * Nc));
    for (int64_t i = 0; i < P * Nc; ++i) {
        if (j->h0) {
            S[i].re = (double)j->h0[((b * H + hh) * P * Nc + i) * 2];
            S[i].im = (double)j->h0[((b * H + hh) * P * Nc + i) * 2 + 1];
        } else { S[i].re = 0.0; S[i].im = 0.0; }
    }
    #define MI_X(t, r) (j->x + (((b * L + (t)) * R + (r)) * H + hh) * P)
    #define MI_BC(T, t, r) (j->T + (((b * L + (t)) * R + (r)) * G + g) * Nc * 2)
    for (int64_t t = 0; t < L; ++t) {
        const double delta = sp((double)j->dt[(b * L + t) * H + hh] + bias);
        const cplx w = {delta * lam.re, delta * lam.im};
        const cplx abar = cexp_(w);
        cplx beta;
        if (bmode == OR_BBAR_ZOH) { cplx f = cphi1(w); beta.re = delta * f.re; beta.im = delta * f.im; }
        else if (bmode == OR_BBAR_DT) { beta.re = delta; beta.im = 0.0; }
        else { beta.re = 1.0; beta.im = 0.0; }
        /* the state update: decay, then every rank's input */
        for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < Nc; ++n) {
                cplx hn = cmul(abar, S[p * Nc + n]);
                for (int64_t r = 0; r < R; ++r) {
                    const float *Bt = MI_BC(B, t, r);
                    const cplx Bn = {(double)Bt[2 * n], (double)Bt[2 * n + 1]};
                    const cplx inp = cmul(beta, Bn);
                    const double xv = (double)MI_X(t, r)[p];
                    hn.re += inp.re * xv;
                    hn.im += inp.im * xv;
                }
                S[p * Nc + n] = hn;
            }
        /* the outputs of every rank from the updated state */
        for (int64_t r = 0; r < R; ++r) {
            const float *Ct = MI_BC(C, t, r);
            double *yt = j->y_out + ((k * L + t) * R + r) * P;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < Nc; ++n) {
                    const double cr = (double)Ct[2 * n], ci = (double)Ct[2 * n + 1];
                    const cplx hn = S[p * Nc + n];
                    acc += conj_c ? (cr * hn.re + ci * hn.im) : (cr * hn.re - ci * hn.im);
                }
                yt[p] = acc + Dh * (double)MI_X(t, r)[p];
            }
        }
    }
    #undef MI_X
    #undef MI_BC
    if (j->hf_out)
        for (int64_t i = 0; i < P * Nc; ++i) {
            j->hf_out[(k * P * Nc + i) * 2] = S[i].re;
            j->hf_out[(k * P * Nc + i) * 2 + 1] = S[i].im;
        }
    free(S);
}

/* ------------------------------------------------------------ threads --- */

typedef struct {
    int kind;               /* 0 S6, 1 SSD, 2 complex, 3 SSD backward, 4 trapezoidal SSD, 5 its backward */
    const void *job;
    int64_t n_units;
    int tid, nthreads;
} worker_arg;

/* ---------------------------------------- Mamba-3 trapezoidal SSD --- */
/*
 * mamba-rs 0.2.1, src/mamba3_siso/gpu/mamba3_gpu.rs (module header; F5b
 * m3_compute_abg; F6 m3_burnin_fwd and its persistent ssm/k/v states): per
 * (b, h), with per-step dt_t, a_t (input-dependent A) and trap_t,
 *   alpha_t = e^{a_t dt_t},  beta_t = alpha_t dt_t (1 - trap_t),  gamma_t = trap_t dt_t
 *   h_t[p,n] = alpha_t h_{t-1}[p,n] + beta_t x_{t-1}[p] k_{t-1}[n] + gamma_t x_t[p] k_t[n]
 *   y[b,t,h,p] = sum_n q_t[n] h_t[p,n] + D[h] x_t[p]
 * with h_{-1} = h0, (x_{-1}, k_{-1}) = (x_prev, k_prev) (each 0 when absent).
 * k, q are per head (B, L, H, N).  Outputs y [n_units][L][P], h_final [n_units][P][N].
 */
typedef struct {
    const float *x, *k, *q, *dt, *a, *trap, *D, *h0, *k_prev, *x_prev;
    int64_t batch, L, H, P, N;
    const int64_t *units;
    int64_t n_units;
    double *y_out, *hf_out;
} trap_job;

static void trap_unit(const trap_job *j, int64_t u)
{
    const int64_t b = j->units[2 * u], hh = j->units[2 * u + 1];
    const int64_t L = j->L, H = j->H, P = j->P, N = j->N;
    const double Dh = j->D ? (double)j->D[hh] : 0.0;
    double *S = (double *)malloc(sizeof(double) * (size_t)(P * N));
    double *xp = (double *)malloc(sizeof(double) * (size_t)P);
    double *kp = (double *)malloc(sizeof(double) * (size_t)N);
    for (int64_t i = 0; i < P * N; ++i) S[i] = j->h0 ? (double)j->h0[(b * H + hh) * P * N + i] : 0.0;
    for (int64_t p = 0; p < P; ++p) xp[p] = j->x_prev ? (double)j->x_prev[(b * H + hh) * P + p] : 0.0;
    for (int64_t n = 0; n < N; ++n) kp[n] = j->k_prev ? (double)j->k_prev[(b * H + hh) * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t o = (b * L + t) * H + hh;
        const double dt = (double)j->dt[o], a = (double)j->a[o], tr = (double)j->trap[o];
        const double alpha = exp(a * dt);
        const double beta = alpha * dt * (1.0 - tr);
        const double gamma = tr * dt;
        const float *xt = j->x + o * P, *kt = j->k + o * N, *qt = j->q + o * N;
        for (int64_t p = 0; p < P; ++p) {
            double *Sp = S + p * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                Sp[n] = alpha * Sp[n] + beta * xp[p] * kp[n] + gamma * (double)xt[p] * (double)kt[n];
                acc += (double)qt[n] * Sp[n];
            }
            j->y_out[(u * L + t) * P + p] = acc + Dh * (double)xt[p];
        }
        for (int64_t p = 0; p < P; ++p) xp[p] = (double)xt[p];
        for (int64_t n = 0; n < N; ++n) kp[n] = (double)kt[n];
    }
    if (j->hf_out) memcpy(j->hf_out + u * P * N, S, sizeof(double) * (size_t)(P * N));
    free(S); free(xp); free(kp);
}

/* ------------------------------------ Mamba-3 trapezoidal backward --- */
/*
 * Gradients of a loss through the trapezoidal recurrence above (mamba-rs
 * 0.2.1 mamba3_gpu.rs pairs F6 with a chunked backward, B6; this is the plain
 * reverse-time chain rule any such scheme must match), given dy = dL/dy and
 * optionally dh_final.  Per unit (b, h), with G_t = dL/dh_t,
 *   G_{L-1} = dh_final + dy_{L-1} (x) q_{L-1},  G_t = dy_t (x) q_t + alpha_{t+1} G_{t+1}
 *   dq_t = h_t^T dy_t;  dx_t = D dy_t + gamma_t G_t k_t + beta_{t+1} G_{t+1} k_t
 *   dk_t = gamma_t G_t^T x_t + beta_{t+1} G_{t+1}^T x_t   (step -1: x_prev, k_prev)
 *   dalpha_t = <G_t, h_{t-1}>, dbeta_t = <G_t, x_{t-1} (x) k_{t-1}>, dgamma_t = <G_t, x_t (x) k_t>
 *   da_t    = dalpha_t dt_t alpha_t + dbeta_t dt_t beta_t
 *   ddt_t   = dalpha_t a_t alpha_t + dbeta_t (1 - trap_t) alpha_t (1 + a_t dt_t) + dgamma_t trap_t
 *   dtrap_t = dgamma_t dt_t - dbeta_t alpha_t dt_t
 *   dD = sum dy . x,  dh0 = alpha_0 G_0.
 * States are recomputed from checkpoints every TRAPB_KSEG steps.  Outputs per
 * unit: dx [L][P], dk, dq [L][N], ddt, da, dtrap [L], dh0 [P][N], dx_prev [P],
 * dk_prev [N], dD [1].
 */
#define TRAPB_KSEG 256
typedef struct {
    const float *x, *k, *q, *dt, *a, *trap, *D, *h0, *k_prev, *x_prev, *dy, *dh_final;
    int64_t batch, L, H, P, N;
    const int64_t *units;
    int64_t n_units;
    double *dx, *dk, *dq, *ddt, *da, *dtrap, *dh0, *dx_prev, *dk_prev, *dD;
} trapb_job;

static void trapb_unit(const trapb_job *j, int64_t u)
{
    const int64_t b = j->units[2 * u], hh = j->units[2 * u + 1];
    const int64_t L = j->L, H = j->H, P = j->P, N = j->N, PN = P * N;
    const double Dh = j->D ? (double)j->D[hh] : 0.0;
    const int64_t nck = (L + TRAPB_KSEG - 1) / TRAPB_KSEG;
    double *ck = (double *)malloc(sizeof(double) * (size_t)(nck * PN));      /* state entering each segment */
    double *Ss = (double *)malloc(sizeof(double) * (size_t)((TRAPB_KSEG + 1) * PN));
    double *Gm = (double *)malloc(sizeof(double) * (size_t)PN);
    double *S = (double *)malloc(sizeof(double) * (size_t)PN);
    double *xm = (double *)malloc(sizeof(double) * (size_t)P);
    double *km = (double *)malloc(sizeof(double) * (size_t)N);
    #define TB_O(t) ((b * L + (t)) * H + hh)
    /* x, k of step t (t = -1: the carried pair) */
    #define TB_X(t, p) ((t) >= 0 ? (double)j->x[TB_O(t) * P + (p)] : (j->x_prev ? (double)j->x_prev[(b * H + hh) * P + (p)] : 0.0))
    #define TB_K(t, n) ((t) >= 0 ? (double)j->k[TB_O(t) * N + (n)] : (j->k_prev ? (double)j->k_prev[(b * H + hh) * N + (n)] : 0.0))
    /* forward: checkpoints */
    for (int64_t i = 0; i < PN; ++i) S[i] = j->h0 ? (double)j->h0[(b * H + hh) * PN + i] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        if (t % TRAPB_KSEG == 0) memcpy(ck + (t / TRAPB_KSEG) * PN, S, sizeof(double) * (size_t)PN);
        const double dt = (double)j->dt[TB_O(t)], a = (double)j->a[TB_O(t)], tr = (double)j->trap[TB_O(t)];
        const double al = exp(a * dt), be = al * dt * (1.0 - tr), ga = tr * dt;
        for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n)
                S[p * N + n] = al * S[p * N + n] + be * TB_X(t - 1, p) * TB_K(t - 1, n) + ga * TB_X(t, p) * TB_K(t, n);
    }
    /* reverse */
    for (int64_t i = 0; i < PN; ++i) Gm[i] = j->dh_final ? (double)j->dh_final[(b * H + hh) * PN + i] : 0.0;
    for (int64_t p = 0; p < P; ++p) xm[p] = 0.0;     /* pending dx of step t from step t+1's beta term */
    for (int64_t n = 0; n < N; ++n) km[n] = 0.0;
    double dD = 0.0;
    for (int64_t c = nck - 1; c >= 0; --c) {
        const int64_t T0 = c * TRAPB_KSEG, T1 = T0 + TRAPB_KSEG < L ? T0 + TRAPB_KSEG : L;
        /* recompute the segment's states: Ss[i] = h_{T0-1+i} */
        memcpy(Ss, ck + c * PN, sizeof(double) * (size_t)PN);
        for (int64_t t = T0; t < T1; ++t) {
            const double dt = (double)j->dt[TB_O(t)], a = (double)j->a[TB_O(t)], tr = (double)j->trap[TB_O(t)];
            const double al = exp(a * dt), be = al * dt * (1.0 - tr), ga = tr * dt;
            const double *Sp = Ss + (t - T0) * PN;
            double *Sn = Ss + (t - T0 + 1) * PN;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    Sn[p * N + n] = al * Sp[p * N + n] + be * TB_X(t - 1, p) * TB_K(t - 1, n) + ga * TB_X(t, p) * TB_K(t, n);
        }
        for (int64_t t = T1 - 1; t >= T0; --t) {
            const int64_t o = TB_O(t);
            const double dt = (double)j->dt[o], a = (double)j->a[o], tr = (double)j->trap[o];
            const double al = exp(a * dt), be = al * dt * (1.0 - tr), ga = tr * dt;
            const float *dyt = j->dy + o * P, *qt = j->q + o * N;
            const double *Ht = Ss + (t - T0 + 1) * PN, *Hp = Ss + (t - T0) * PN;
            /* G_t = G_t (carried, already alpha_{t+1} G_{t+1} + dh_final) + dy_t (x) q_t */
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) Gm[p * N + n] += (double)dyt[p] * (double)qt[n];
            /* dq_t */
            for (int64_t n = 0; n < N; ++n) {
                double s = 0.0;
                for (int64_t p = 0; p < P; ++p) s += Ht[p * N + n] * (double)dyt[p];
                j->dq[(u * L + t) * N + n] = s;
            }
            /* dalpha, dbeta, dgamma */
            double dal = 0.0, dbe = 0.0, dga = 0.0;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) {
                    const double g = Gm[p * N + n];
                    dal += g * Hp[p * N + n];
                    dbe += g * TB_X(t - 1, p) * TB_K(t - 1, n);
                    dga += g * TB_X(t, p) * TB_K(t, n);
                }
            /* dx_t, dk_t: own gamma term plus the pending beta term of step t+1 */
            for (int64_t p = 0; p < P; ++p) {
                double s = 0.0;
                for (int64_t n = 0; n < N; ++n) s += Gm[p * N + n] * TB_K(t, n);
                j->dx[(u * L + t) * P + p] = Dh * (double)dyt[p] + ga * s + xm[p];
                dD += (double)dyt[p] * TB_X(t, p);
            }
            for (int64_t n = 0; n < N; ++n) {
                double s = 0.0;
                for (int64_t p = 0; p < P; ++p) s += Gm[p * N + n] * TB_X(t, p);
                j->dk[(u * L + t) * N + n] = ga * s + km[n];
            }
            /* this step's beta term, for step t-1 (or the carried pair) */
            for (int64_t p = 0; p < P; ++p) {
                double s = 0.0;
                for (int64_t n = 0; n < N; ++n) s += Gm[p * N + n] * TB_K(t - 1, n);
                xm[p] = be * s;
            }
            for (int64_t n = 0; n < N; ++n) {
                double s = 0.0;
                for (int64_t p = 0; p < P; ++p) s += Gm[p * N + n] * TB_X(t - 1, p);
                km[n] = be * s;
            }
            j->da[u * L + t] = dal * dt * al + dbe * dt * be;
            j->ddt[u * L + t] = dal * a * al + dbe * (1.0 - tr) * al * (1.0 + a * dt) + dga * tr;
            j->dtrap[u * L + t] = dga * dt - dbe * al * dt;
            /* carry to step t-1 */
            for (int64_t i = 0; i < PN; ++i) Gm[i] *= al;
        }
    }
    memcpy(j->dh0 + u * PN, Gm, sizeof(double) * (size_t)PN);
    memcpy(j->dx_prev + u * P, xm, sizeof(double) * (size_t)P);
    memcpy(j->dk_prev + u * N, km, sizeof(double) * (size_t)N);
    j->dD[u] = dD;
    #undef TB_O
    #undef TB_X
    #undef TB_K
    free(ck); free(Ss); free(Gm); free(S); free(xm); free(km);
}

/* ------------------------------------------------------- SSD backward --- */
/*
 * Gradients of a loss L through the SSD recurrence above, given dy = dL/dy
 * and optionally dh_final = dL/dS_{L-1}: the reverse-time chain rule of the
 * sequential recurrence (the page's ssd.js pairs its forward with a chunk
 * backward; this is the plain definition that any such scheme must match).
 * Per unit (b, h), with G_t = dL/dS_t (P x N):
 *   G_{L-1} = dh_final + dy_{L-1} (x) C_{L-1};  G_{t-1} = e^{a_t} G_t + dy_{t-1} (x) C_{t-1}
 *   dx_t[p]  = D dy_t[p] + sigma_t sum_n G_t[p,n] B_t[n]
 *   dB_t[n] += sigma_t sum_p x_t[p] G_t[p,n]        (summed over the heads of group g)
 *   dC_t[n] += sum_p dy_t[p] S_t[p,n]              (likewise)
 *   da_t     = e^{a_t} sum_{p,n} G_t[p,n] S_{t-1}[p,n],  dsigma_t = sum_{p,n} G_t x_t[p] B_t[n]
 *   ddelta_t = da_t A + dsigma_t dsigma/ddelta,  dA += da_t delta_t + dsigma_t dsigma/dA
 *   (DT: dsigma/ddelta = 1, dsigma/dA = 0;  ZOH: e^{a}, delta^2 phi1'(a);  ONE: 0, 0)
 *   ddt_t = ddelta_t sigmoid(dt + dt_bias);  dA_log = A dA;  dD = sum dy x;  dh0 = e^{a_0} G_0
 * S_{t-1} is re-run from checkpoints every KSEG steps (S_{-1} = h0), so memory
 * stays at (L/KSEG + KSEG) P N doubles per unit.
 * Outputs per unit k (double): dx [L][P], dB, dC [L][N] (this head's share),
 * ddt [L], dh0 [P][N], and the scalars dA_log, dD, ddt_bias of this (b, h).
 */
#define SSDB_KSEG 256

typedef struct {
    const float *x, *dt, *dt_bias, *A_log, *B, *C, *D, *h0, *dy, *dhf;
    int64_t batch, L, H, P, N, G;
    uint32_t flags;
    const int64_t *units;
    int64_t n_units;
    double *dx, *dB, *dC, *ddt, *dh0, *dA_log, *dD, *ddtb;
} ssdb_job;

static double dphi1(double z);
static double sigm(double x);

static void ssdb_unit(const ssdb_job *j, int64_t k)
{
    const int64_t b = j->units[2 * k], hh = j->units[2 * k + 1];
    const int64_t L = j->L, H = j->H, P = j->P, N = j->N, G = j->G, PN = P * N;
    const int64_t g = hh * G / H;
    const int mode = (int)(j->flags & OR_BBAR_MASK);
    const double A = -exp((double)j->A_log[hh]);
    const double bias = j->dt_bias ? (double)j->dt_bias[hh] : 0.0;
    const double Dh = j->D ? (double)j->D[hh] : 0.0;
    const int64_t nseg = (L + SSDB_KSEG - 1) / SSDB_KSEG;
    double *ck = (double *)malloc(sizeof(double) * (size_t)(nseg * PN));   /* S entering segment */
    double *Ss = (double *)malloc(sizeof(double) * (size_t)((SSDB_KSEG + 1) * PN));
    double *Gm = (double *)malloc(sizeof(double) * (size_t)PN);
    double *ut = (double *)malloc(sizeof(double) * (size_t)P);
    /* per-step scalars */
    #define SSDB_X(t) (j->x + ((b * L + (t)) * H + hh) * P)
    #define SSDB_B(t) (j->B + ((b * L + (t)) * G + g) * N)
    #define SSDB_C(t) (j->C + ((b * L + (t)) * G + g) * N)
    #define SSDB_DY(t) (j->dy + ((b * L + (t)) * H + hh) * P)
    /* forward: checkpoints */
    double *S = Ss;
    for (int64_t i = 0; i < PN; ++i) S[i] = j->h0 ? (double)j->h0[(b * H + hh) * PN + i] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        if (t % SSDB_KSEG == 0) memcpy(ck + (t / SSDB_KSEG) * PN, S, sizeof(double) * (size_t)PN);
        const double delta = sp((double)j->dt[(b * L + t) * H + hh] + bias);
        const double a = delta * A;
        const double sigma = mode == OR_BBAR_DT ? delta : (mode == OR_BBAR_ZOH ? delta * phi1(a) : 1.0);
        const double dec = exp(a);
        for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n)
                S[p * N + n] = dec * S[p * N + n] + sigma * (double)SSDB_X(t)[p] * (double)SSDB_B(t)[n];
    }
    /* backward */
    for (int64_t i = 0; i < PN; ++i) Gm[i] = j->dhf ? (double)j->dhf[(b * H + hh) * PN + i] : 0.0;
    double dA = 0.0, dD = 0.0, ddtb = 0.0;
    for (int64_t sgi = nseg - 1; sgi >= 0; --sgi) {
        const int64_t t0 = sgi * SSDB_KSEG, t1 = (t0 + SSDB_KSEG < L) ? t0 + SSDB_KSEG : L;
        /* Ss[0] = S_{t0-1}, Ss[i+1] = S_{t0+i} */
        memcpy(Ss, ck + sgi * PN, sizeof(double) * (size_t)PN);
        for (int64_t t = t0; t < t1; ++t) {
            const double delta = sp((double)j->dt[(b * L + t) * H + hh] + bias);
            const double a = delta * A;
            const double sigma = mode == OR_BBAR_DT ? delta : (mode == OR_BBAR_ZOH ? delta * phi1(a) : 1.0);
            const double dec = exp(a);
            const double *Sp = Ss + (t - t0) * PN;
            double *Sn = Ss + (t - t0 + 1) * PN;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    Sn[p * N + n] = dec * Sp[p * N + n] + sigma * (double)SSDB_X(t)[p] * (double)SSDB_B(t)[n];
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double xdt = (double)j->dt[(b * L + t) * H + hh] + bias;
            const double delta = sp(xdt);
            const double a = delta * A;
            double sigma, dsd, dsa;
            if (mode == OR_BBAR_DT) { sigma = delta; dsd = 1.0; dsa = 0.0; }
            else if (mode == OR_BBAR_ZOH) { sigma = delta * phi1(a); dsd = exp(a); dsa = delta * delta * dphi1(a); }
            else { sigma = 1.0; dsd = 0.0; dsa = 0.0; }
            const double dec = exp(a);
            const float *xt = SSDB_X(t), *Bt = SSDB_B(t), *Ct = SSDB_C(t), *dyt = SSDB_DY(t);
            const double *St = Ss + (t - t0 + 1) * PN, *Sprev = Ss + (t - t0) * PN;
            /* G_t: add this step's output cotangent */
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) Gm[p * N + n] += (double)dyt[p] * (double)Ct[n];
            double *dBt = j->dB + (k * L + t) * N, *dCt = j->dC + (k * L + t) * N;
            for (int64_t n = 0; n < N; ++n) {
                double sb = 0.0, sc = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    sb += (double)xt[p] * Gm[p * N + n];
                    sc += (double)dyt[p] * St[p * N + n];
                }
                dBt[n] = sigma * sb;
                dCt[n] = sc;
            }
            double dsig = 0.0, da = 0.0;
            for (int64_t p = 0; p < P; ++p) {
                double s = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    s += Gm[p * N + n] * (double)Bt[n];
                    da += Gm[p * N + n] * Sprev[p * N + n];
                }
                ut[p] = s;
                dsig += (double)xt[p] * s;
                j->dx[(k * L + t) * P + p] = Dh * (double)dyt[p] + sigma * s;
                dD += (double)dyt[p] * (double)xt[p];
            }
            da *= dec;
            const double ddelta = da * A + dsig * dsd;
            dA += da * delta + dsig * dsa;
            const double ddt = ddelta * sigm(xdt);
            j->ddt[k * L + t] = ddt;
            ddtb += ddt;
            /* G_{t-1} part carried from G_t */
            for (int64_t i = 0; i < PN; ++i) Gm[i] *= dec;
        }
    }
    memcpy(j->dh0 + k * PN, Gm, sizeof(double) * (size_t)PN);
    j->dA_log[k] = dA * A;
    j->dD[k] = dD;
    j->ddtb[k] = ddtb;
    #undef SSDB_X
    #undef SSDB_B
    #undef SSDB_C
    #undef SSDB_DY
    free(ck); free(Ss); free(Gm); free(ut);
}

static void *worker(void *p)
{
    const worker_arg *w = (const worker_arg *)p;
    for (int64_t k = w->tid; k < w->n_units; k += w->nthreads) {
        if (w->kind == 0) s6_unit((const s6_job *)w->job, k);
        else if (w->kind == 1) ssd_unit((const ssd_job *)w->job, k);
        else if (w->kind == 2) cssd_unit((const cssd_job *)w->job, k);
        else if (w->kind == 3) ssdb_unit((const ssdb_job *)w->job, k);
        else if (w->kind == 4) trap_unit((const trap_job *)w->job, k);
        else if (w->kind == 5) trapb_unit((const trapb_job *)w->job, k);
        else mimo_unit((const mimo_job *)w->job, k);
    }
    return NULL;
}

static void run_units(int kind, const void *job, int64_t n_units, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n_units) nthreads = (int)(n_units > 0 ? n_units : 1);
    pthread_t th[256];
    worker_arg args[256];
    for (int i = 0; i < nthreads; ++i) {
        args[i].kind = kind; args[i].job = job; args[i].n_units = n_units;
        args[i].tid = i; args[i].nthreads = nthreads;
    }
    if (nthreads == 1) { worker(&args[0]); return; }
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &args[i]);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------ exports --- */

void oracle_s6_fwd(const float *u, const float *dt, const float *dt_bias, const float *A_log,
                   const float *B, const float *C, const float *D, const float *h0,
                   int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, uint32_t flags,
                   const int64_t *units, int64_t n_units, double *y_out, double *hf_out,
                   int nthreads)
{
    s6_job j = {u, dt, dt_bias, A_log, B, C, D, h0, batch, L, d_inner, d_state, flags,
                units, n_units, y_out, hf_out};
    run_units(0, &j, n_units, nthreads);
}

/*
 * The S6 recurrence with B and C per group of channels (per channel when
 * ngroups = d_inner): the variable B, C of the selective scan page's header
 * taken per channel instead of shared (builderforce-memory-engine
 * selective_scan.js header comment), with channel d reading group
 * d * ngroups / d_inner.  B, C (batch, L, ngroups, d_state).
 */
void oracle_s6_grouped_fwd(const float *u, const float *dt, const float *dt_bias, const float *A_log,
                           const float *B, const float *C, const float *D, const float *h0,
                           int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                           uint32_t flags, const int64_t *units, int64_t n_units, double *y_out,
                           double *hf_out, int nthreads)
{
    s6_job j = {u, dt, dt_bias, A_log, B, C, D, h0, batch, L, d_inner, d_state, flags,
                units, n_units, y_out, hf_out};
    j.G = ngroups;
    run_units(0, &j, n_units, nthreads);
}

/*
 * Mamba-1 layer around the scan (builderforce-memory-engine conv1d.ts header
 * and conv1d_forward; mamba-rs 0.4.0 forward.rs F4a conv1d burn-in with fused
 * SiLU and carried conv state, F4d scan, F4e gating):
 *   u[b,t,d] = SiLU(sum_{k<K} conv_w[d,k] x[b,t-k,d] + conv_b[d]),
 *              x[b,t',d] for t' < 0 from conv_state[b,d,K-1+t'] (oldest first) or 0
 *   y        = the S6 scan of u (D u included), times SiLU(z[b,t,d]) when z is given
 * u_out [n_units][L], cs_out [n_units][K-1] (x of the last K-1 steps, the state
 * a next call carries) may be NULL.
 */
void oracle_s6_layer_fwd(const float *x, const float *conv_w, const float *conv_b,
                         const float *conv_state, const float *z, const float *dt,
                         const float *dt_bias, const float *A_log, const float *B, const float *C,
                         const float *D, const float *h0, int64_t batch, int64_t L, int64_t d_inner,
                         int64_t d_state, int64_t d_conv, uint32_t flags, const int64_t *units,
                         int64_t n_units, double *y_out, double *hf_out, double *u_out, double *cs_out,
                         int nthreads)
{
    s6_job j = {x, dt, dt_bias, A_log, B, C, D, h0, batch, L, d_inner, d_state, flags,
                units, n_units, y_out, hf_out, conv_w, conv_b, conv_state, z, d_conv, u_out, cs_out};
    run_units(0, &j, n_units, nthreads);
}

void oracle_ssd_fwd(const float *x, const float *dt, const float *dt_bias, const float *A_log,
                    const float *B, const float *C, const float *D, const float *h0,
                    int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                    int64_t ngroups, uint32_t flags, const int64_t *units, int64_t n_units,
                    double *y_out, double *hf_out, int nthreads)
{
    ssd_job j = {x, dt, dt_bias, A_log, B, C, D, h0, batch, L, nheads, headdim, d_state, ngroups,
                 flags, units, n_units, y_out, hf_out};
    run_units(1, &j, n_units, nthreads);
}

void oracle_cssd_fwd(const float *x, const float *dt, const float *dt_bias, const float *A_log,
                     const float *B, const float *C, const float *D, const float *h0,
                     int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t n_complex,
                     int64_t ngroups, uint32_t flags, const int64_t *units, int64_t n_units,
                     double *y_out, double *hf_out, int nthreads)
{
    cssd_job j = {x, dt, dt_bias, A_log, B, C, D, h0, batch, L, nheads, headdim, n_complex, ngroups,
                  flags, units, n_units, y_out, hf_out};
    run_units(2, &j, n_units, nthreads);
}

void oracle_cssd_mimo_fwd(const float *x, const float *dt, const float *dt_bias, const float *A_log,
                          const float *B, const float *C, const float *D, const float *h0,
                          int64_t batch, int64_t L, int64_t rank, int64_t nheads, int64_t headdim,
                          int64_t n_complex, int64_t ngroups, uint32_t flags, const int64_t *units,
                          int64_t n_units, double *y_out, double *hf_out, int nthreads)
{
    mimo_job j = {x, dt, dt_bias, A_log, B, C, D, h0, batch, L, rank, nheads, headdim, n_complex, ngroups,
                  flags, units, n_units, y_out, hf_out};
    run_units(6, &j, n_units, nthreads);
}

/* ------------------------------------------------------- S6 backward --- */
/*
 * Gradient of a loss L with respect to every input of the S6 forward scan,
 * given dy = dL/dy (batch, L, d_inner) and optionally dL/dh_final.  This is
 * the chain rule applied to the sequential recurrence above, step by step in
 * reverse time (the reverse scan the S6 page lays out in backward_scan of
 * selective_scan.js, completed with the terms that page leaves out: beta's
 * dependence on A and the sums over channels for the shared B and C):
 *
 *   g_t      = dL/dh_t = g_{t+1} Abar_{t+1} + C_t dy_t   (g_L = dL/dh_final)
 *   dC_t[n] += dy_t[d] h_t[n]                 (summed over d)
 *   dB_t[n] += g_t beta_t u_t[d]              (summed over d)
 *   du_t[d]  = D dy_t + sum_n g_t beta_t B_t[n]
 *   ddelta_t = sum_n g_t (h_{t-1} dAbar/ddelta + B_t u_t dbeta/ddelta)
 *   dA[d,n] += g_t (h_{t-1} dAbar/dA + B_t u_t dbeta/dA)   (summed over b, t)
 *   Abar = e^{delta A}:  dAbar/ddelta = A Abar,  dAbar/dA = delta Abar
 *   ZOH beta = delta phi1(delta A): dbeta/ddelta = Abar, dbeta/dA = delta^2 phi1'(delta A)
 *   DT beta = delta: 1, 0;   ONE beta = 1: 0, 0
 *   ddt = ddelta * sigmoid(dt + dt_bias) (softplus' = sigmoid); ddt_bias = sum ddt
 *   dA_log = dA * A (A = -exp(A_log));  dD[d] = sum dy u;  dh0 = g_0 Abar_0
 *
 * Units are (b, d) for b in [b_lo, b_hi), d in [d_lo, d_hi); sums over b or d
 * run over those ranges only, so a caller can take complete sums by passing
 * full ranges.  Outputs are double:
 *   du, ddt [nb][L][nd];  dB, dC [nb][L][N];  dA_log [nd][N];
 *   dD, ddt_bias [nd];  dh0 [nb][nd][N]
 */

/* phi1'(z) = (e^z (z - 1) + 1)/z^2 = (expm1(z)(z - 1) + z)/z^2, phi1'(0) = 1/2;
 * below |z| = 1e-3 its Taylor series sum_m (m+1) z^m/(m+2)! (to z^4). */
static double dphi1(double z)
{
    if (fabs(z) < 1e-3) return 0.5 + z * (1.0 / 3.0 + z * (1.0 / 8.0 + z * (1.0 / 30.0 + z / 144.0)));
    return (expm1(z) * (z - 1.0) + z) / (z * z);
}

static double sigm(double x)
{
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    const double e = exp(x);
    return e / (1.0 + e);
}

typedef struct {
    const float *u, *dt, *dt_bias, *A_log, *B, *C, *D, *h0, *dy, *dhf;
    int64_t batch, L, Dm, N, b_lo, b_hi, d_lo, d_hi;
    uint32_t flags;
    double *du, *ddt, *dB, *dC, *dA_log, *dD, *ddtb, *dh0;   /* shared outputs */
    int64_t G;   /* B, C per group of channels (batch, L, G, N), channel d in group d*G/Dm; 0: shared */
} s6b_job;

typedef struct {
    const s6b_job *j;
    int tid, nthreads;
    double *dB, *dC, *dA, *dD, *ddtb;   /* this thread's partial sums */
} s6b_arg;

static void s6b_unit(const s6b_job *j, s6b_arg *w, int64_t b, int64_t d)
{
    const int64_t L = j->L, Dm = j->Dm, N = j->N;
    const int64_t G = j->G > 0 ? j->G : 1, gi = d * G / Dm;   /* this channel's B, C row */
    const int64_t nd = j->d_hi - j->d_lo, bi = b - j->b_lo, di = d - j->d_lo;
    const int mode = (int)(j->flags & OR_BBAR_MASK);
    double *A = (double *)malloc(sizeof(double) * (size_t)N);
    double *g = (double *)malloc(sizeof(double) * (size_t)N);
    double *h = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));   /* h[t+1] = h_t, h[0] = h0 */
    for (int64_t n = 0; n < N; ++n) {
        A[n] = -exp((double)j->A_log[d * N + n]);
        h[n] = j->h0 ? (double)j->h0[(b * Dm + d) * N + n] : 0.0;
        g[n] = j->dhf ? (double)j->dhf[(b * Dm + d) * N + n] : 0.0;
    }
    const double bias = j->dt_bias ? (double)j->dt_bias[d] : 0.0;
    const double Dd = j->D ? (double)j->D[d] : 0.0;
    /* forward, keeping every state */
    for (int64_t t = 0; t < L; ++t) {
        const int64_t e = (b * L + t) * Dm + d;
        const double delta = sp((double)j->dt[e] + bias);
        const double uu = (double)j->u[e];
        const float *Bt = j->B + ((b * L + t) * G + gi) * N;
        for (int64_t n = 0; n < N; ++n) {
            const double z = delta * A[n];
            double beta;
            if (mode == OR_BBAR_ZOH) beta = delta * phi1(z);
            else if (mode == OR_BBAR_DT) beta = delta;
            else beta = 1.0;
            h[(t + 1) * N + n] = exp(z) * h[t * N + n] + beta * (double)Bt[n] * uu;
        }
    }
    /* reverse */
    for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t e = (b * L + t) * Dm + d;
        const double x = (double)j->dt[e] + bias;
        const double delta = sp(x);
        const double uu = (double)j->u[e];
        const double dyv = (double)j->dy[e];
        const float *Bt = j->B + ((b * L + t) * G + gi) * N;
        const float *Ct = j->C + ((b * L + t) * G + gi) * N;
        double ddelta = 0.0, duv = Dd * dyv;
        for (int64_t n = 0; n < N; ++n) {
            const double z = delta * A[n];
            const double Ab = exp(z);
            double beta, bD, bA;
            if (mode == OR_BBAR_ZOH) { beta = delta * phi1(z); bD = Ab; bA = delta * delta * dphi1(z); }
            else if (mode == OR_BBAR_DT) { beta = delta; bD = 1.0; bA = 0.0; }
            else { beta = 1.0; bD = 0.0; bA = 0.0; }
            g[n] += (double)Ct[n] * dyv;
            const double hp = h[t * N + n], ht = h[(t + 1) * N + n];
            const double Bu = (double)Bt[n] * uu;
            w->dC[((bi * L + t) * G + gi) * N + n] += dyv * ht;
            w->dB[((bi * L + t) * G + gi) * N + n] += g[n] * beta * uu;
            duv += g[n] * beta * (double)Bt[n];
            ddelta += g[n] * (hp * A[n] * Ab + Bu * bD);
            w->dA[di * N + n] += g[n] * (hp * delta * Ab + Bu * bA);
            g[n] *= Ab;
        }
        const double ddt = ddelta * sigm(x);
        j->ddt[(bi * L + t) * nd + di] = ddt;
        j->du[(bi * L + t) * nd + di] = duv;
        w->ddtb[di] += ddt;
        w->dD[di] += dyv * uu;
    }
    if (j->dh0)
        for (int64_t n = 0; n < N; ++n) j->dh0[(bi * nd + di) * N + n] = g[n];
    free(A);
    free(g);
    free(h);
}

static void *s6b_worker(void *p)
{
    s6b_arg *w = (s6b_arg *)p;
    const s6b_job *j = w->j;
    const int64_t nd = j->d_hi - j->d_lo, nu = (j->b_hi - j->b_lo) * nd;
    for (int64_t k = w->tid; k < nu; k += w->nthreads)
        s6b_unit(j, w, j->b_lo + k / nd, j->d_lo + k % nd);
    return NULL;
}

static void s6_bwd_run(const float *u, const float *dt, const float *dt_bias, const float *A_log,
                       const float *B, const float *C, const float *D, const float *h0,
                       const float *dy, const float *dh_final,
                       int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                       uint32_t flags, int64_t b_lo, int64_t b_hi, int64_t d_lo, int64_t d_hi,
                       double *du, double *ddt, double *dB, double *dC, double *dA_log, double *dD,
                       double *ddt_bias, double *dh0, int nthreads)
{
    const int64_t nb = b_hi - b_lo, nd = d_hi - d_lo, N = d_state;
    s6b_job j = {u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, batch, L, d_inner, d_state,
                 b_lo, b_hi, d_lo, d_hi, flags, du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0, ngroups};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nb * nd) nthreads = (int)(nb * nd > 0 ? nb * nd : 1);
    const size_t nbc = (size_t)(nb * L * (ngroups > 0 ? ngroups : 1) * N);
    s6b_arg args[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) {
        args[i].j = &j; args[i].tid = i; args[i].nthreads = nthreads;
        args[i].dB = (double *)calloc(nbc, sizeof(double));
        args[i].dC = (double *)calloc(nbc, sizeof(double));
        args[i].dA = (double *)calloc((size_t)(nd * N), sizeof(double));
        args[i].dD = (double *)calloc((size_t)nd, sizeof(double));
        args[i].ddtb = (double *)calloc((size_t)nd, sizeof(double));
    }
    if (nthreads == 1) s6b_worker(&args[0]);
    else {
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, s6b_worker, &args[i]);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    }
    memset(dB, 0, nbc * sizeof(double));
    memset(dC, 0, nbc * sizeof(double));
    memset(dA_log, 0, (size_t)(nd * N) * sizeof(double));
    memset(dD, 0, (size_t)nd * sizeof(double));
    memset(ddt_bias, 0, (size_t)nd * sizeof(double));
    for (int i = 0; i < nthreads; ++i) {   /* fixed order: the result does not depend on timing */
        for (size_t k = 0; k < nbc; ++k) { dB[k] += args[i].dB[k]; dC[k] += args[i].dC[k]; }
        for (int64_t k = 0; k < nd * N; ++k) dA_log[k] += args[i].dA[k];
        for (int64_t k = 0; k < nd; ++k) { dD[k] += args[i].dD[k]; ddt_bias[k] += args[i].ddtb[k]; }
        free(args[i].dB); free(args[i].dC); free(args[i].dA); free(args[i].dD); free(args[i].ddtb);
    }
    for (int64_t di = 0; di < nd; ++di)   /* dA -> dA_log: dA/dA_log = A */
        for (int64_t n = 0; n < N; ++n)
            dA_log[di * N + n] *= -exp((double)A_log[(d_lo + di) * N + n]);
}


void oracle_s6_bwd(const float *u, const float *dt, const float *dt_bias, const float *A_log,
                   const float *B, const float *C, const float *D, const float *h0,
                   const float *dy, const float *dh_final,
                   int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, uint32_t flags,
                   int64_t b_lo, int64_t b_hi, int64_t d_lo, int64_t d_hi,
                   double *du, double *ddt, double *dB, double *dC, double *dA_log, double *dD,
                   double *ddt_bias, double *dh0, int nthreads)
{
    s6_bwd_run(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, batch, L, d_inner, d_state, 0, flags,
               b_lo, b_hi, d_lo, d_hi, du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0, nthreads);
}

/* The backward of oracle_s6_grouped_fwd: dB, dC (nb, L, ngroups, N) summed over each
 * group's channels in the unit range; the rest as oracle_s6_bwd. */
void oracle_s6_grouped_bwd(const float *u, const float *dt, const float *dt_bias, const float *A_log,
                           const float *B, const float *C, const float *D, const float *h0,
                           const float *dy, const float *dh_final,
                           int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, int64_t ngroups,
                           uint32_t flags, int64_t b_lo, int64_t b_hi, int64_t d_lo, int64_t d_hi,
                           double *du, double *ddt, double *dB, double *dC, double *dA_log, double *dD,
                           double *ddt_bias, double *dh0, int nthreads)
{
    s6_bwd_run(u, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, batch, L, d_inner, d_state, ngroups, flags,
               b_lo, b_hi, d_lo, d_hi, du, ddt, dB, dC, dA_log, dD, ddt_bias, dh0, nthreads);
}

/* elementary functions, exported so the tests can pin them on their own */
void oracle_ssd_bwd(const float *x, const float *dt, const float *dt_bias, const float *A_log,
                    const float *B, const float *C, const float *D, const float *h0,
                    const float *dy, const float *dh_final,
                    int64_t batch, int64_t L, int64_t nheads, int64_t headdim, int64_t d_state,
                    int64_t ngroups, uint32_t flags, const int64_t *units, int64_t n_units,
                    double *dx, double *dB, double *dC, double *ddt, double *dh0,
                    double *dA_log, double *dD, double *ddt_bias, int nthreads)
{
    ssdb_job j = {x, dt, dt_bias, A_log, B, C, D, h0, dy, dh_final, batch, L, nheads, headdim,
                  d_state, ngroups, flags, units, n_units, dx, dB, dC, ddt, dh0, dA_log, dD, ddt_bias};
    run_units(3, &j, n_units, nthreads);
}

void oracle_trap_fwd(const float *x, const float *k, const float *q, const float *dt, const float *a,
                     const float *trap, const float *D, const float *h0, const float *k_prev,
                     const float *x_prev, int64_t batch, int64_t L, int64_t nheads, int64_t headdim,
                     int64_t d_state, const int64_t *units, int64_t n_units, double *y_out,
                     double *hf_out, int nthreads)
{
    trap_job j = {x, k, q, dt, a, trap, D, h0, k_prev, x_prev, batch, L, nheads, headdim, d_state,
                  units, n_units, y_out, hf_out};
    run_units(4, &j, n_units, nthreads);
}

/* ------------------------------------- Mamba-3 data-dependent rotation --- */
/*
 * mamba-rs 0.2.1, src/mamba3_siso/gpu/mamba3_gpu.rs, F5 (m3_angle_dt_fwd_seq:
 * angle * dt accumulated step by step per batch row, carried in angle_state)
 * and F4e+f (rope_fwd: k, q rotated by the accumulated angles).  Per (b, h)
 * and angle j < n_angles:
 *   theta_t[j] = angle_state[b,h,j] + sum_{s<=t} angles[b,s,j] dt[b,s,h]
 *   (k'[2j], k'[2j+1]) = (k[2j] cos theta - k[2j+1] sin theta,
 *                         k[2j] sin theta + k[2j+1] cos theta)
 * and the same for q; components 2 n_angles .. d_state-1 are unchanged.
 * state_out[b,h,j] = theta_{L-1}[j] (angle_state when L == 0).
 * k, q, k_out, q_out (B, L, H, N); angles (B, L, n_angles); dt (B, L, H);
 * angle_state, state_out (B, H, n_angles).
 */
void oracle_trap_rotate(const float *k, const float *q, const float *angles, const float *dt,
                        const float *angle_state, int64_t batch, int64_t L, int64_t nheads,
                        int64_t d_state, int64_t n_angles, double *k_out, double *q_out,
                        double *state_out)
{
    const int64_t H = nheads, N = d_state, NA = n_angles;
    double *th = (double *)malloc(sizeof(double) * (size_t)(NA > 0 ? NA : 1));
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t j = 0; j < NA; ++j)
                th[j] = angle_state ? (double)angle_state[(b * H + h) * NA + j] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const double d = (double)dt[(b * L + t) * H + h];
                const int64_t o = ((b * L + t) * H + h) * N;
                for (int64_t j = 0; j < NA; ++j) th[j] += (double)angles[(b * L + t) * NA + j] * d;
                for (int64_t n = 0; n < N; ++n) { k_out[o + n] = (double)k[o + n]; q_out[o + n] = (double)q[o + n]; }
                for (int64_t j = 0; j < NA; ++j) {
                    const double c = cos(th[j]), sn = sin(th[j]);
                    const double k0 = (double)k[o + 2 * j], k1 = (double)k[o + 2 * j + 1];
                    const double q0 = (double)q[o + 2 * j], q1 = (double)q[o + 2 * j + 1];
                    k_out[o + 2 * j] = k0 * c - k1 * sn;
                    k_out[o + 2 * j + 1] = k0 * sn + k1 * c;
                    q_out[o + 2 * j] = q0 * c - q1 * sn;
                    q_out[o + 2 * j + 1] = q0 * sn + q1 * c;
                }
            }
            for (int64_t j = 0; j < NA; ++j) state_out[(b * H + h) * NA + j] = th[j];
        }
    free(th);
}

void oracle_trap_bwd(const float *x, const float *k, const float *q, const float *dt, const float *a,
                     const float *trap, const float *D, const float *h0, const float *k_prev,
                     const float *x_prev, const float *dy, const float *dh_final, int64_t batch, int64_t L,
                     int64_t nheads, int64_t headdim, int64_t d_state, const int64_t *units, int64_t n_units,
                     double *dx, double *dk, double *dq, double *ddt, double *da, double *dtrap, double *dh0,
                     double *dx_prev, double *dk_prev, double *dD, int nthreads)
{
    trapb_job j = {x, k, q, dt, a, trap, D, h0, k_prev, x_prev, dy, dh_final, batch, L, nheads, headdim,
                   d_state, units, n_units, dx, dk, dq, ddt, da, dtrap, dh0, dx_prev, dk_prev, dD};
    run_units(5, &j, n_units, nthreads);
}

double oracle_softplus(double x) { return sp(x); }
double oracle_phi1(double z) { return phi1(z); }
double oracle_dphi1(double z) { return dphi1(z); }
