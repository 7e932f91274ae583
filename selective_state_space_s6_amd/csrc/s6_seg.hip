// s6_seg.hip -- the segmented S6 forward scan, for long sequences over few
// channels (a batch of one or two rows of a Mamba-1 layer at long context),
// where the sequential walk of s6_scan.hip would leave most compute units idle.
//
// The recurrence h_t = Abar_t h_{t-1} + b_t is a chain of affine maps, and the
// maps compose associatively: running (P1, h1) and then (P2, h2) is
// (P2 P1, P2 h1 + h2) -- the earlier map first (selective_scan.js forward_scan
// carries its tiles this way; its printed combine applies the earlier decay to
// the later input, which is the reverse order).  So:
//  1. every segment but the last runs from a zero state (s6_scan_kernel PASS 1),
//     leaving its local final state h_loc and its sum of delta; the segment's
//     decay is P = exp(A * sum), the product of its steps' Abar;
//  2. s6_seg_carry_kernel scans the pairs (0, h0), (P_0, h_loc_0), ... with that
//     rule across the lanes of a wave (DPP row shifts within 16-lane rows, row
//     broadcasts across them), giving the state entering every segment;
//  3. every segment runs again from its entering state and writes y
//     (s6_scan_kernel PASS 3); the last one writes h_final.
// The first pass repeats the arithmetic of all but the last segment without the
// output sum: about 1.8x the work of the walk for 8x to 64x the parallel width.
#include "s6_kernel.hpp"

namespace ssm {
namespace {

constexpr int64_t kSegMinLen = 512;   // shortest segment worth a second pass
constexpr int64_t kSegFill = 768;     // blocks that fill the chip (3 per compute unit)
constexpr int64_t kSegMax = 64;       // segments of one carry scan (the lanes of a wave)

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// One step of an inclusive scan over the lanes of a wave: the lane composes the
// pair that DPP control CTRL brings from an earlier lane (earlier map first) with
// its own.  Lanes the control does not reach, or rows outside ROWS, get the
// identity pair (1, 0) from update_dpp's old value and keep their own.
template <int CTRL, int ROWS>
__device__ __forceinline__ void carry_step(float &P, float &h) {
    const float Pe = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, P), CTRL, ROWS, 0xf, false));
    const float he = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, h), CTRL, ROWS, 0xf, false));
    h = fmaf(P, he, h);   // the later decay applied to the earlier state, plus the later state
    P = P * Pe;
}

// One wave per (b, d, n): lane 0 holds (0, h0) (the entering state), lane j >= 1
// the pair of segment j - 1, lanes past the segments the identity.  After the
// scan, lane j holds the state entering segment j.
__global__ void __launch_bounds__(256)
s6_seg_carry_kernel(const float *A_log, const float *h0, const float *h_loc, const double *dsum, float *h_in,
                    int64_t batch, int64_t Dm, int64_t N, int64_t nseg) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool uok = unit < batch * Dm * N;            // uniform over the wave
    const int64_t uu = uok ? unit : 0;
    const int64_t n = uu % N, d = (uu / N) % Dm, b = uu / (N * Dm);
    float P = 1.0f, h = 0.0f;
    if (uok && lane < nseg) {
        if (lane == 0) {
            P = 0.0f;
            h = h0 ? h0[(b * Dm + d) * N + n] : 0.0f;
        } else {
            const int64_t s = lane - 1;
            // log2 of the segment's decay, exp(A * sum of delta), formed in double
            const double A = -fmin(exp((double)A_log[d * N + n]), 1e300);
            const double x = A * 1.4426950408889634 * dsum[(b * (nseg - 1) + s) * Dm + d];
            P = exp2_fast((float)fmax(x, -1.0e4));
            h = h_loc[((b * (nseg - 1) + s) * Dm + d) * N + n];
        }
    }
    carry_step<0x111, 0xf>(P, h);   // row_shr:1
    carry_step<0x112, 0xf>(P, h);   // row_shr:2
    carry_step<0x114, 0xf>(P, h);   // row_shr:4
    carry_step<0x118, 0xf>(P, h);   // row_shr:8: each 16-lane row scanned
    carry_step<0x142, 0xa>(P, h);   // row_bcast:15 into rows 1 and 3
    carry_step<0x143, 0xc>(P, h);   // row_bcast:31 into rows 2 and 3
    if (uok && lane < nseg) h_in[((b * nseg + lane) * Dm + d) * N + n] = h;
}

}  // namespace

S6SegPlan s6_seg_plan(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state) {
    S6SegPlan pl{1, L, 0};
    if (d_state > 16 || L < 2 * kSegMinLen) return pl;
    const int64_t G = d_state <= 1 ? 1 : d_state <= 2 ? 2 : d_state <= 4 ? 4 : d_state <= 8 ? 8 : 16;
    const int64_t CW = kThreads / G;
    const int64_t blocks = batch * ((d_inner + CW - 1) / CW);
    if (4 * blocks > kSegFill) return pl;      // a quarter of the chip or more: walk in sequence
    int64_t nseg = std::min(std::min(kSegMax, kSegFill / blocks), L / kSegMinLen);
    if (nseg < 2) return pl;
    const int64_t seg_len = ((L + nseg - 1) / nseg + kT - 1) / kT * kT;   // whole 16-step tiles
    nseg = (L + seg_len - 1) / seg_len;
    if (nseg < 2) return pl;
    pl.nseg = nseg;
    pl.seg_len = seg_len;
    pl.ws_bytes = align256((size_t)(batch * (nseg - 1) * d_inner * d_state) * sizeof(float)) +
                  align256((size_t)(batch * (nseg - 1) * d_inner) * sizeof(double)) +
                  align256((size_t)(batch * nseg * d_inner * d_state) * sizeof(float));
    return pl;
}

hipError_t launch_s6_segmented(const S6Args &a, const S6SegPlan &pl, hipStream_t stream, const char **kernel_name) {
    S6Kp p{};
    p.u = a.u; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log; p.B = a.B; p.C = a.C;
    p.D = a.D; p.y = a.y; p.h0 = nullptr; p.h_final = a.h_final;
    p.batch = a.batch; p.L = a.L; p.Dm = a.d_inner; p.N = a.d_state;
    p.seg_len = pl.seg_len; p.nseg = pl.nseg;
    char *ws = static_cast<char *>(a.workspace);
    const size_t n_loc = align256((size_t)(a.batch * (pl.nseg - 1) * a.d_inner * a.d_state) * sizeof(float));
    const size_t n_sum = align256((size_t)(a.batch * (pl.nseg - 1) * a.d_inner) * sizeof(double));
    p.h_loc = reinterpret_cast<float *>(ws);
    p.dsum = reinterpret_cast<double *>(ws + n_loc);
    float *h_in = reinterpret_cast<float *>(ws + n_loc + n_sum);
    p.h_in = h_in;
    const int mode = (int)(a.flags & 0x3u);
    *kernel_name = "s6_scan_kernel (segment states)";
    hipError_t e = a.bf16 ? launch_shape_seg<uint16_t, 1>(p, mode, stream) : launch_shape_seg<float, 1>(p, mode, stream);
    if (e != hipSuccess) return e;
    *kernel_name = "s6_seg_carry_kernel";
    const int64_t units = a.batch * a.d_inner * a.d_state;
    hipLaunchKernelGGL(s6_seg_carry_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream,
                       a.A_log, a.h0, p.h_loc, p.dsum, h_in, a.batch, a.d_inner, a.d_state, pl.nseg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    *kernel_name = "s6_scan_kernel (segment scan)";
    return a.bf16 ? launch_shape_seg<uint16_t, 3>(p, mode, stream) : launch_shape_seg<float, 3>(p, mode, stream);
}

}  // namespace ssm
