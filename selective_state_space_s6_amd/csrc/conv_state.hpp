// conv_state.hpp -- the carried state of a causal depthwise conv: after a call
// over L steps, state_out[b, c, j] = x at time L-(K-1)+j, taken from the old
// state when that time is before 0.  One thread per (b, c) reads everything it
// needs before it writes, and the kernel runs after the conv that reads the old
// state, so the state may be updated in place.
#pragma once
#include "device_common.hpp"

namespace ssm {
namespace {

constexpr int kMaxConvTaps = 4;   // longest causal convolution

template <typename TIN>
__global__ void __launch_bounds__(256)
conv_state_out_kernel(const TIN *x, const float *cs_in, float *cs_out, int64_t batch, int64_t L,
                      int64_t Dc, int K) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= batch * Dc) return;
    const int64_t b = i / Dc, c = i % Dc;
    float v[kMaxConvTaps - 1];
#pragma unroll
    for (int j = 0; j < kMaxConvTaps - 1; ++j) {
        if (j >= K - 1) break;
        const int64_t tt = L - (K - 1) + j;
        v[j] = tt >= 0 ? In<TIN>::ld(x, (b * L + tt) * Dc + c)
                       : (cs_in ? cs_in[i * (K - 1) + (K - 1) + tt] : 0.0f);
    }
#pragma unroll
    for (int j = 0; j < kMaxConvTaps - 1; ++j) {
        if (j >= K - 1) break;
        cs_out[i * (K - 1) + j] = v[j];
    }
}

template <typename TIN>
void launch_conv_state_out(const TIN *x, const float *cs_in, float *cs_out, int64_t batch, int64_t L,
                           int64_t Dc, int K, hipStream_t stream) {
    const int64_t n = batch * Dc;
    hipLaunchKernelGGL(conv_state_out_kernel<TIN>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       x, cs_in, cs_out, batch, L, Dc, K);
}

}  // namespace
}  // namespace ssm
