"""Shared helpers of the GPU parity tests: run the HIP path through the
binding, run the oracle on the same inputs, compare with the north-star
metric.  Nothing here does scan arithmetic."""
import numpy as np
import torch

import oracle
import synth

TOL_F32 = 1e-4     # max relative error, fp32 inputs
TOL_BF16 = 2e-2    # max relative error, bf16 inputs with fp32 state
# Backward pass (fp32 arithmetic on the exact input values, bf16 or fp32): its outputs
# are sums over up to d_inner channels (dB, dC), batch*L steps (dA_log) or 16 states
# (du, ddt) of products of fp32 states and cotangents, each carrying a relative rounding
# error eps of a few ulp (~3e-7) accumulated over the recurrence's memory.  A K-term sum of
# random-sign terms has rms ~ sqrt(K)|term| and error ~ eps sqrt(K)|term|, so near a zero
# of the result the metric's floor 0.01*rms turns it into ~eps*z/0.01 with z ~ 5 the largest
# deviate among 1e5-1e7 elements: ~2e-4.  A plain fp32 computation of the same gradients
# (numpy, each op rounded) scores 1.3e-4 to 1e-3 at the Mamba-1 layer shape.
TOL_BWD = 1e-3


def lib():
    import selective_state_space_s6_amd as s
    return s


def report(name, **errs):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)


def gpu_s6(inp, device, flags):
    t = inp.torch(device)
    y, hf = lib().ssm_s6_scan_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                  t["h0"], flags=flags, return_final=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), hf.cpu().numpy()


def gpu_ssd(inp, device, flags, chunk_len):
    t = inp.torch(device)
    y, hf = lib().ssd_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"],
                                     t["D"], t["h0"], chunk_len=chunk_len, flags=flags,
                                     return_final=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), hf.cpu().numpy()


def gpu_trap(inp, device, chunk_len=64):
    t = inp.torch(device)
    y, hf = lib().ssd_trap_chunk_scan_fwd(t["x"], t["k"], t["q"], t["dt"], t["a"], t["trap"], t["D"],
                                          t["h0"], t["k_prev"], t["x_prev"], chunk_len=chunk_len,
                                          return_final=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), hf.cpu().numpy()


def gpu_cssd(inp, device, flags, chunk_len):
    t = inp.torch(device)
    y, hf = lib().ssd_cplx_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"],
                                          t["D"], t["h0"], chunk_len=chunk_len, flags=flags,
                                          return_final=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), hf.cpu().numpy()


def sample_units(rng, n0, n1, k):
    idx = rng.choice(n0 * n1, size=min(k, n0 * n1), replace=False)
    return np.stack([idx // n1, idx % n1], 1)
