#!/usr/bin/env python3
"""Benchmark of the forward selective-scan hot path on one MI355X.

A step is one call of the scan entry point over one batch of synthetic input
already resident in HBM (for S6: softplus, discretisation, recurrence, state
reduction and skip term, all inside one kernel; for the chunked SSD paths, the
segment-state, state-pass and chunk-scan kernels of one call).  The headline is
the largest single-GPU workload, the long-context SSD (batch 2, L 32768, 80
heads x 64, N 128, 8 groups, bf16 in, fp32 state and output); every one of the
five workloads (S6 tiny, S6 at a Mamba-1 layer shape, SSD at a Mamba-2 shape,
long-context SSD, complex SSD) gets a full line under "configs", each with its
roofline and the fp64 oracle timed on the host cores; the other paths (Mamba-3,
per-channel B/C, the layer, decode steps, backward passes, the segmented long
S6) are under "secondary".  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-secondary] [--no-cpu]

--workload NAME measures that one workload alone in the headline schema (the
profiling runs use it); NAME copy_1gib is a plain 1 GiB device copy, the
reference for scaling the HBM byte counters.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6   # dense bf16 MFMA (no sparsity), TFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3   # dense fp32 MFMA
# the roof of each chunked path, priced at the dtype its contractions run in
MFMA_PEAKS = {
    "ssd": (BF16_MFMA_PEAK_TFLOPS, "dense bf16 MFMA (model flops of the chunked decomposition)"),
    "trap": (BF16_MFMA_PEAK_TFLOPS, "dense bf16 MFMA (model flops of the chunked decomposition)"),
    "cssd": (FP32_MFMA_PEAK_TFLOPS, "dense fp32 MFMA (model flops of the complex chunked decomposition)"),
    "cssd_mimo": (FP32_MFMA_PEAK_TFLOPS, "dense fp32 MFMA (the complex model over L x rank rows)"),
    "ssd_bwd": (FP32_MFMA_PEAK_TFLOPS, "dense fp32 MFMA (the walks' contraction work, in 16x16x4 MFMA units)"),
    "trap_bwd": (FP32_MFMA_PEAK_TFLOPS, "dense fp32 MFMA (the walks' contraction work, in 16x16x4 MFMA units)"),
}
FP32_VALU_PEAK_TFLOPS = 78.6     # 256 CU x 64 lanes x 2 flop (FMA) x 2.4 GHz, non-packed fp32
# fp32 VALU issue: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz lane-slots/s (a wave64 op takes 4 cycles)
VALU_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9
# one ZOH state update (b, t, d, n) of the S6 kernel: x = dl*A, exp2 (half rate: 2 slots), the
# (Abar-1)/A form, the 3-FMA series for phi1 and delta*p, compare + select, B*u, the state
# update h + beta (A h + B u) (two FMAs), y += C*h, and the partial-sum add of the reduction
# over states: 14 single-rate ops + the exp = 16 issue slots (counted: 15.8 VALU instructions
# per update at the Mamba-1 shape)
S6_SLOTS_PER_UPDATE = 16
S6_FLOPS_PER_UPDATE = 9          # the method's flops per update (the series is the exp's cost)
# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled
# by the same counters on a 1 GiB device copy (bench.py --workload copy_1gib); each entry is
# valid only while the sha1 of the kernels' sources matches (profiles/*.md, "HBM traffic")
TRAFFIC = {
    "s6_mamba1": {
        "src_sha1": "a79736759aeaa1fce6cc1bbc7762eaa5f3d16967",
        "bytes": 308664790
    },
    "ssd_mamba2": {
        "src_sha1": "5784943de805795f1dd6d85d75f4db3f1adf3b43",
        "bytes": 502900386
    },
    "ssd_long": {
        "src_sha1": "5784943de805795f1dd6d85d75f4db3f1adf3b43",
        "bytes": 3622451415
    },
    "cssd_mamba3": {
        "src_sha1": "ae7254e078839793bbf80b24c4a75b00f4c40ee9",
        "bytes": 1106262528
    }
}
# adjoint update of one (b, t, d, n) in ZOH mode: g += C dy, dh terms of du, ddt, dB, dC, dA
# (products and fmas, 24 flops) plus the recomputed Abar, beta, phi1' (not counted again)
S6_BWD_FLOPS_PER_UPDATE = 24
N_ROTATE = 3                     # input copies rotated between steps (> Infinity Cache)
CPU_SAMPLE_WALL_S = 1.0          # wall time the SSD-type oracle samples aim at (16 host threads)
# (--copies 1 for the counter runs, where each dispatch is read on its own)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def s6_model(d):
    """Algorithmic bytes and operations of one S6 call: u, dt read and y written per
    (b, t, d); B, C read per (b, t, n); A_log, D, dt_bias and the final state once."""
    B, L, D, N = d["batch"], d["L"], d["d_inner"], d["d_state"]
    elems = B * L * D
    isz = 4
    bytes_ = elems * (isz + 4 + 4) + 2 * B * L * N * isz + D * N * 4 + 2 * D * 4 + B * D * N * 4
    ops = elems * N * S6_FLOPS_PER_UPDATE   # per (b,t,d,n) state update
    return elems, bytes_, ops


def s6_pc_model(d):
    """S6 with B, C per group of channels: u, dt read and y written per (b, t, d); B, C
    read once per (b, t, group, n); the same state updates as s6_model."""
    B, L, D, N, G = d["batch"], d["L"], d["d_inner"], d["d_state"], d["ngroups"]
    elems = B * L * D
    bytes_ = elems * 12 + 2 * B * L * G * N * 4 + D * N * 4 + 2 * D * 4 + B * D * N * 4
    return elems, bytes_, elems * N * S6_FLOPS_PER_UPDATE


def s6_layer_model(d):
    """The fused layer: read x, z, dt (fp32), B, C, the conv state and h0; write y, h_final
    and the conv state.  Operations: the scan's state updates (the conv, SiLU and gate
    are ~0.1 % of them at N = 16, not counted)."""
    B, L, D, N, K = d["batch"], d["L"], d["d_inner"], d["d_state"], d["d_conv"]
    elems = B * L * D
    bytes_ = elems * 4 * 4 + 2 * B * L * N * 4 + 2 * B * D * (K - 1) * 4 + 2 * B * D * N * 4 + D * N * 4
    return elems, bytes_, elems * N * S6_FLOPS_PER_UPDATE


def s6_bwd_model(d):
    """Algorithmic bytes of one S6 backward call: read u, dt, dy, B, C, write du, ddt,
    dB, dC, dA_log, dD, ddt_bias, dh0 (and read dh_final); ops: one forward state
    update (to have h) plus the adjoint update per (b, t, d, n)."""
    B, L, D, N = d["batch"], d["L"], d["d_inner"], d["d_state"]
    G = d.get("ngroups") or 1          # B, C and dB, dC per group of channels
    elems = B * L * D
    bytes_ = elems * 4 * 5 + 4 * B * L * G * N * 4 + 2 * B * D * N * 4 + D * N * 8 + 3 * D * 4
    ops = elems * N * (S6_FLOPS_PER_UPDATE + S6_BWD_FLOPS_PER_UPDATE)
    return elems, bytes_, ops


def ssd_bwd_model(d):
    """Algorithmic bytes of one SSD backward call (read x, B, C, dt, dy; write dx, ddt, dB, dC)
    and the contraction work of its walks, in units of 16x16x4 fp32 MFMAs (2048 flops each):
    per (batch, head) and 32-step chunk each of the three walks 3P/4 + 3N/4 + PN/16 (656 at
    P = 64, N = 128), and the two state-only walks PN/32 each over all segments but one.  (The
    gradient-state updates of walks R1 and R2 do their PN/16 share on bf16 MFMAs, the fp32
    operand split into three bf16 terms; the work counted is the contraction's, not those
    three passes.)"""
    B, L, H, P, N, G = d["batch"], d["L"], d["nheads"], d["headdim"], d["d_state"], d["ngroups"]
    elems = B * L * H * P
    bytes_ = (elems * 2 + 2 * B * L * G * N * 2 + B * L * H * 4 + elems * 4 + elems * 4 +
              B * L * H * 4 + 2 * B * L * G * N * 4)
    nseg = d.get("nseg", 1)
    units = B * H * (-(-L // 32))
    walk = 3 * P // 4 + 3 * N // 4 + P * N // 16
    mfmas = units * 3 * walk + units * (P * N // 16) * (nseg - 1) // nseg
    return elems, bytes_, mfmas * 2048


def ssd_model(d):
    B, L, H, P, N, G, Q = (d["batch"], d["L"], d["nheads"], d["headdim"], d["d_state"], d["ngroups"],
                           d["chunk_len"])
    elems = B * L * H * P
    nc = -(-L // Q)
    bytes_ = elems * 2 + 2 * B * L * G * N * 2 + B * L * H * 4 + elems * 4 + B * H * P * N * 4
    if d.get("carry"):            # the entering state is read too
        bytes_ += B * H * P * N * 4
    # dense-square MFMA flops: C.B^T once per (b, chunk, group); (G o L) X, chunk states and
    # state->output per (b, chunk, head)
    flops = 2 * B * nc * (G * Q * Q * N + H * (Q * Q * P + 2 * Q * P * N))
    return elems, bytes_, flops


def trap_model(d):
    """Mamba-3 trapezoidal SSD: bf16 x, per-head bf16 k and q, fp32 dt, a, trap in; fp32 y and
    final state out.  Flops as the SSD with one group per head (k.q^T per head)."""
    B, L, H, P, N, Q = d["batch"], d["L"], d["nheads"], d["headdim"], d["d_state"], d["chunk_len"]
    elems = B * L * H * P
    nc = -(-L // Q)
    bytes_ = elems * 2 + 2 * B * L * H * N * 2 + 3 * B * L * H * 4 + elems * 4 + B * H * P * N * 4
    if d.get("carry"):            # the entering state and the previous x, k are read too
        bytes_ += B * H * P * N * 4 + B * H * (P + N) * 2
    flops = 2 * B * nc * H * (Q * Q * N + Q * Q * P + 2 * Q * P * N)
    return elems, bytes_, flops


def trap_rot_model(d):
    """Rotation of k and q: read k, q (bf16), angles, dt and the angle state; write k, q and
    the final angles.  Elements are (b, t, h, head channel) as for the scan it feeds."""
    B, L, H, P, N, NA = d["batch"], d["L"], d["nheads"], d["headdim"], d["d_state"], d["n_angles"]
    elems = B * L * H * P
    bytes_ = 4 * B * L * H * N * 2 + B * L * NA * 4 + B * L * H * 4 + 2 * B * H * NA * 4
    return elems, bytes_, 0


def conv_model(d):
    """Causal conv1d: read x, write y (dtype size each), weights, bias and the states."""
    B, L, Cc, K = d["batch"], d["L"], d["channels"], d["d_conv"]
    isz = 2 if d.get("bf16") else 4
    elems = B * L * Cc
    return elems, elems * isz * 2 + Cc * (K + 1) * 4 + 2 * B * Cc * (K - 1) * 4, elems * (2 * K + 4)


def cssd_model(d):
    """Algorithmic bytes (x, y fp32; B, C complex per group; dt; the final state) and the
    real-equivalent flops of the complex chunked decomposition, per (b, chunk): the complex
    C.B^T once per group as two real GEMMs with K = 2 N_c (8 Q^2 N_c), and per head Re(M) X
    (2 Q^2 P), the complex chunk state from real x (two real GEMMs, 4 Q P N_c) and Re(C h)
    (one real GEMM with K = 2 N_c, 4 Q P N_c)."""
    B, L, H, P, Nc, G, Q = (d["batch"], d["L"], d["nheads"], d["headdim"], d["n_complex"],
                            d["ngroups"], d["chunk_len"])
    elems = B * L * H * P
    bytes_ = elems * 4 * 2 + 2 * B * L * G * Nc * 8 + B * L * H * 4 + B * H * P * Nc * 8
    nc = -(-L // Q)
    flops = B * nc * (G * 8 * Q * Q * Nc + H * (2 * Q * Q * P + 8 * Q * P * Nc))
    return elems, bytes_, flops


def mimo_model(d):
    """The complex SSD's model over L x rank rows (every row is an input and an output row);
    elems counts output values, batch * L * rank * H * P."""
    R = d["rank"]
    dd = dict(d, L=d["L"] * R)
    elems, bytes_, flops = cssd_model(dd)
    bytes_ -= (R - 1) * d["batch"] * d["L"] * d["nheads"] * 4      # dt is read once per step
    return elems, bytes_, flops


def make_runner(name, dev):
    """Returns (step_fn(i), dims, kernel names) with N_ROTATE resident input copies."""
    import numpy as np
    import torch
    import selective_state_space_s6_amd as lib
    import synth
    # name suffixes: _bwd (the backward), _bwd_saved (the backward reading the forward's saved
    # states), _fwd_save (the forward that saves them)
    if name == "copy_1gib":       # the reference copy for the HBM byte counters
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)

        def step(i):
            dst.copy_(src)
        return step, {"bytes": 2 << 30}, {"kind": "copy", "dtype": "f32"}, ["copy"]
    walk = name.endswith("_walk")      # the S6 scan without a workspace: the sequential walk
    if walk:
        name = name[: -len("_walk")]
    saved = name.endswith("_bwd_saved")
    save = name.endswith("_fwd_save")
    if saved:
        name = name[: -len("_saved")]
    if save:
        name = name[: -len("_fwd_save")]
    bwd = name.endswith("_bwd")
    if bwd:
        name = name[: -len("_bwd")]
    w = dict(synth.WORKLOADS[name])
    kind = w["kind"]
    copies = []
    for r in range(N_ROTATE):
        inp = synth.workload_inputs(name, seed=(r,))
        copies.append(inp.torch(dev))
        dims = inp.dims
    if kind == "s6" and bwd:
        d = dims
        for r, t in enumerate(copies):
            dy, dhf = synth.s6_cotangents(d["batch"], d["L"], d["d_inner"], d["d_state"], seed=(r,))
            t["dy"], t["dhf"] = torch.from_numpy(dy).to(dev), torch.from_numpy(dhf).to(dev)
        gsh = (d["ngroups"],) if d.get("ngroups") else ()
        shapes = dict(du=(d["batch"], d["L"], d["d_inner"]), ddt=(d["batch"], d["L"], d["d_inner"]),
                      dB=(d["batch"], d["L"], *gsh, d["d_state"]), dC=(d["batch"], d["L"], *gsh, d["d_state"]),
                      dA_log=(d["d_inner"], d["d_state"]), dD=(d["d_inner"],),
                      ddt_bias=(d["d_inner"],), dh0=(d["batch"], d["d_inner"], d["d_state"]))
        out = {k: torch.empty(v, dtype=torch.float32, device=dev) for k, v in shapes.items()}
        ws = torch.empty(lib.ssm_s6_scan_bwd_workspace_size(d["batch"], d["L"], d["d_inner"],
                                                            d["d_state"]), dtype=torch.uint8, device=dev)
        if d.get("ngroups"):       # B, C per group of channels
            ws = torch.empty(lib.ssm_s6_scan_grouped_bwd_workspace_size(d["batch"], d["L"], d["d_inner"],
                                                                        d["d_state"], d["ngroups"]),
                             dtype=torch.uint8, device=dev)

            if saved:  # each copy's states, saved once by the forward outside the timed region
                for t in copies:
                    t["ck"] = lib.ssm_s6_scan_grouped_fwd_save(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"],
                                                               t["C"], t["D"], None)[2]

                def step(i):
                    t = copies[i % N_ROTATE]
                    lib.ssm_s6_scan_grouped_bwd_saved(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"],
                                                      t["D"], None, t["dy"], t["dhf"], t["ck"], out=out,
                                                      workspace=ws)
            else:
                def step(i):
                    t = copies[i % N_ROTATE]
                    lib.ssm_s6_scan_grouped_bwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                                None, t["dy"], t["dhf"], out=out, workspace=ws)
            w["kind"] = "s6_bwd"
            return step, dims, w, ["s6_grouped_bwd_kernel", "s6_grouped_bwd_reduce"]
        if saved:      # each copy's states, saved once by the forward outside the timed region
            for t in copies:
                t["ck"] = lib.ssm_s6_scan_fwd_save(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"],
                                                   t["D"], None)[2]

            def step(i):
                t = copies[i % N_ROTATE]
                lib.ssm_s6_scan_bwd_saved(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                          None, t["dy"], t["dhf"], t["ck"], out=out, workspace=ws)
        else:
            def step(i):
                t = copies[i % N_ROTATE]
                lib.ssm_s6_scan_bwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                    None, t["dy"], t["dhf"], out=out, workspace=ws)
        w["kind"] = "s6_bwd"
        return step, dims, w, ["s6_bwd_kernel", "s6_bwd_reduce_kernel"]
    if kind == "s6" and save:
        t0 = copies[0]
        y = torch.empty_like(t0["u"], dtype=torch.float32)
        hf = torch.empty((dims["batch"], dims["d_inner"], dims["d_state"]), dtype=torch.float32, device=dev)
        ck = torch.empty((dims["batch"], (dims["L"] + 15) // 16, dims["d_inner"], dims["d_state"]),
                         dtype=torch.float32, device=dev)

        if dims.get("ngroups"):    # B, C per group of channels
            def step(i):
                t = copies[i % N_ROTATE]
                lib.ssm_s6_scan_grouped_fwd_save(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"],
                                                 t["D"], None, y=y, h_final=hf, checkpoints=ck)
            w["kind"] = "s6_pc_save"
            return step, dims, w, ["s6_grouped_kernel"]

        def step(i):
            t = copies[i % N_ROTATE]
            lib.ssm_s6_scan_fwd_save(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                     None, y=y, h_final=hf, checkpoints=ck)
        w["kind"] = "s6_save"
        return step, dims, w, ["s6_scan_kernel"]
    if kind == "conv":
        t0 = copies[0]
        y = torch.empty_like(t0["x"])
        so = torch.empty_like(t0["state"])

        def step(i):
            t = copies[i % N_ROTATE]
            lib.ssm_causal_conv1d_fwd(t["x"], t["w"], t["bias"], t["state"], silu=w["silu"], y=y, state_out=so)
        dims = dict(dims, bf16=w["dtype"] == "bf16")
        return step, dims, w, ["conv1d_kernel", "conv_state_out_kernel"]
    if kind == "s6_layer":
        t0 = copies[0]
        y = torch.empty(t0["x"].shape, dtype=torch.float32, device=dev)
        states = [(t["h0"].clone(), t["conv_state"].clone()) for t in copies]

        def step(i):
            t = copies[i % N_ROTATE]
            h, cs = states[i % N_ROTATE]     # carried in place, as a decode loop does
            lib.ssm_s6_fused_fwd(t["x"], t["conv_w"], t["conv_b"], t["dt"], t["dt_bias"], t["A_log"], t["B"],
                                 t["C"], t["D"], h, cs, t["z"], y=y, h_final=h, conv_state_out=cs)
        return step, dims, w, (["s6_step4_kernel"] if dims["L"] == 1 else ["s6_scan_kernel", "s6_conv_state_kernel"])
    if kind == "s6" and w.get("ngroups"):
        t0 = copies[0]
        y = torch.empty_like(t0["u"], dtype=torch.float32)
        hf = torch.empty((dims["batch"], dims["d_inner"], dims["d_state"]), dtype=torch.float32, device=dev)

        def step(i):
            t = copies[i % N_ROTATE]
            lib.ssm_s6_scan_grouped_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                        None, y=y, h_final=hf)
        w["kind"] = "s6_pc"
        return step, dims, w, ["s6_grouped_kernel"]
    if kind == "s6":
        t0 = copies[0]
        y = torch.empty_like(t0["u"], dtype=torch.float32)
        hf = torch.empty((dims["batch"], dims["d_inner"], dims["d_state"]), dtype=torch.float32, device=dev)
        nws = 0 if walk else lib.ssm_s6_scan_fwd_workspace_size(dims["batch"], dims["L"], dims["d_inner"],
                                                                dims["d_state"])
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None

        def step(i):
            t = copies[i % N_ROTATE]
            lib.ssm_s6_scan_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                None, y=y, h_final=hf, workspace=ws)
        if ws is not None:
            dims = dict(dims, segmented=True)
            return step, dims, w, ["s6_scan_kernel (segment states)", "s6_seg_carry_kernel",
                                   "s6_scan_kernel (segment scan)"]
        return step, dims, w, ["s6_scan_kernel"]
    if kind == "trap" and bwd:
        d = dims
        for r, t in enumerate(copies):
            rng = np.random.default_rng([9, r])
            t["dy"] = torch.from_numpy(rng.standard_normal(
                (d["batch"], d["L"], d["nheads"], d["headdim"]), dtype=np.float32)).to(dev)
            t["dhf"] = torch.from_numpy(rng.standard_normal(
                (d["batch"], d["nheads"], d["headdim"], d["d_state"]), dtype=np.float32)).to(dev)
        ws = torch.empty(lib.ssd_trap_chunk_scan_bwd_workspace_size(
            d["batch"], d["L"], d["nheads"], d["headdim"], d["d_state"], w["chunk_len"]), dtype=torch.uint8, device=dev)
        out = {}

        def step(i):
            t = copies[i % N_ROTATE]
            g = lib.ssd_trap_chunk_scan_bwd(t["x"], t["k"], t["q"], t["dt"], t["a"], t["trap"], t["D"], None, None,
                                            None, t["dy"], t["dhf"], chunk_len=w["chunk_len"], out=out or None,
                                            workspace=ws)
            out.update({k: v for k, v in g.items() if v is not None})
        w["kind"] = "trap_bwd"
        return step, dims, w, ["ssdb_walk_f", "ssdb_walk_r1", "ssdb_walk_r2", "ssdb_pass_f", "ssdb_pass_r",
                               "ssdb_reduce_heads", "ssdb_scal", "ssdb_final",
                               "trapb_prev_kernel", "trapb_chain_kernel"]
    if kind == "ssd" and bwd:
        d = dims
        for r, t in enumerate(copies):
            rng = np.random.default_rng([5, r])
            t["dy"] = torch.from_numpy(rng.standard_normal(
                (d["batch"], d["L"], d["nheads"], d["headdim"]), dtype=np.float32)).to(dev)
            t["dhf"] = torch.from_numpy(rng.standard_normal(
                (d["batch"], d["nheads"], d["headdim"], d["d_state"]), dtype=np.float32)).to(dev)
        ws = torch.empty(lib.ssd_chunk_scan_bwd_workspace_size(
            d["batch"], d["L"], d["nheads"], d["headdim"], d["d_state"], d["ngroups"], w["chunk_len"]),
            dtype=torch.uint8, device=dev)
        out = {}

        def step(i):
            t = copies[i % N_ROTATE]
            g = lib.ssd_chunk_scan_bwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                       None, t["dy"], t["dhf"], chunk_len=w["chunk_len"],
                                       out=out or None, workspace=ws)
            out.update(g)
        w["kind"] = "ssd_bwd"
        return step, dims, w, ["ssdb_walk_f", "ssdb_walk_r1", "ssdb_walk_r2", "ssdb_pass_f", "ssdb_pass_r",
                               "ssdb_reduce_heads", "ssdb_scal", "ssdb_final"]
    if kind == "trap_rot":
        t0 = copies[0]
        angs = []
        for r in range(N_ROTATE):
            ang, st = synth.rotation_inputs(dims["batch"], dims["L"], dims["nheads"], w["n_angles"],
                                            seed=(r,))
            angs.append((torch.from_numpy(ang).to(dev), torch.from_numpy(st).to(dev)))
        ko, qo = torch.empty_like(t0["k"]), torch.empty_like(t0["q"])
        so = torch.empty_like(angs[0][1])
        ws = torch.empty(max(1, lib.ssd_trap_rotate_qk_workspace_size(
            dims["batch"], dims["L"], dims["nheads"], dims["d_state"], w["n_angles"])),
            dtype=torch.uint8, device=dev)

        def step(i):
            t = copies[i % N_ROTATE]
            ang, st = angs[i % N_ROTATE]
            lib.ssd_trap_rotate_qk(t["k"], t["q"], ang, t["dt"], st, k=ko, q=qo, angle_state_out=so,
                                   workspace=ws)
        dims = dict(dims, n_angles=w["n_angles"])
        return step, dims, w, ["trap_rot_sums4_kernel", "trap_rot_apply4_kernel"]
    if kind == "trap":
        t0 = copies[0]
        y = torch.empty(t0["x"].shape, dtype=torch.float32, device=dev)
        hf = torch.empty((dims["batch"], dims["nheads"], dims["headdim"], dims["d_state"]),
                         dtype=torch.float32, device=dev)
        ws = torch.empty(lib.ssd_trap_chunk_scan_fwd_workspace_size(
            dims["batch"], dims["L"], dims["nheads"], dims["headdim"], dims["d_state"],
            w["chunk_len"]), dtype=torch.uint8, device=dev)

        if w.get("carry"):            # decode: the state carried in place, previous x, k passed
            states = [t["h0"].clone() for t in copies]

            def step(i):
                t = copies[i % N_ROTATE]
                h = states[i % N_ROTATE]
                lib.ssd_trap_chunk_scan_fwd(t["x"], t["k"], t["q"], t["dt"], t["a"], t["trap"], t["D"], h,
                                            t["k_prev"], t["x_prev"], chunk_len=w["chunk_len"], y=y,
                                            h_final=h, workspace=ws)
            return step, dims, w, ["ssd_trap_step_kernel"]

        def step(i):
            t = copies[i % N_ROTATE]
            lib.ssd_trap_chunk_scan_fwd(t["x"], t["k"], t["q"], t["dt"], t["a"], t["trap"], t["D"],
                                        None, None, None, chunk_len=w["chunk_len"], y=y, h_final=hf,
                                        workspace=ws)
        return step, dims, w, ["ssd_state_kernel", "ssd_pass_kernel", "ssd_scan_kernel"]
    if kind == "ssd":
        t0 = copies[0]
        y = torch.empty(t0["x"].shape, dtype=torch.float32, device=dev)
        hf = torch.empty((dims["batch"], dims["nheads"], dims["headdim"], dims["d_state"]),
                         dtype=torch.float32, device=dev)
        ws = torch.empty(lib.ssd_chunk_scan_fwd_workspace_size(
            dims["batch"], dims["L"], dims["nheads"], dims["headdim"], dims["d_state"],
            dims["ngroups"], w["chunk_len"]), dtype=torch.uint8, device=dev)

        if w.get("carry"):            # decode: the state carried in place
            states = [t["h0"].clone() for t in copies]

            def step(i):
                t = copies[i % N_ROTATE]
                h = states[i % N_ROTATE]
                lib.ssd_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                       h, chunk_len=w["chunk_len"], y=y, h_final=h, workspace=ws)
            return step, dims, w, ["ssd_step_kernel"]

        def step(i):
            t = copies[i % N_ROTATE]
            lib.ssd_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                   None, chunk_len=w["chunk_len"], y=y, h_final=hf, workspace=ws)
        return step, dims, w, ["ssd_state_kernel", "ssd_pass_kernel", "ssd_scan_kernel"]
    t0 = copies[0]
    y = torch.empty(t0["x"].shape, dtype=torch.float32, device=dev)
    hf = torch.empty((dims["batch"], dims["nheads"], dims["headdim"], dims["n_complex"], 2),
                     dtype=torch.float32, device=dev)
    if kind == "cssd_mimo":
        ws = torch.empty(lib.ssd_cplx_mimo_chunk_scan_fwd_workspace_size(
            dims["batch"], dims["L"], dims["rank"], dims["nheads"], dims["headdim"], dims["n_complex"],
            dims["ngroups"], w["chunk_len"]), dtype=torch.uint8, device=dev)

        def step(i):
            t = copies[i % N_ROTATE]
            lib.ssd_cplx_mimo_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                             None, chunk_len=w["chunk_len"], y=y, h_final=hf, workspace=ws)
        return step, dims, w, ["cssd_prep_kernel", "cssd_state_kernel", "cssd_pass_kernel", "cssd_scan_kernel"]
    ws = torch.empty(lib.ssd_cplx_chunk_scan_fwd_workspace_size(
        dims["batch"], dims["L"], dims["nheads"], dims["headdim"], dims["n_complex"],
        dims["ngroups"], w["chunk_len"]), dtype=torch.uint8, device=dev)

    def step(i):
        t = copies[i % N_ROTATE]
        lib.ssd_cplx_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"],
                                    None, chunk_len=w["chunk_len"], y=y, h_final=hf, workspace=ws)
    return step, dims, w, ["cssd_prep_kernel", "cssd_state_kernel", "cssd_pass_kernel", "cssd_scan_kernel"]


def time_steps(step, steps, warmup):
    """Warmup, then time exactly `steps` steps between two device synchronisations.
    Per-step HIP events on the launch stream give the per-launch durations."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record()
        step(warmup + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in evs]   # ms
    return wall, per


def graph_us_per_step(step, n=32, replays=20):
    """Per-step time of n steps captured in one HIP graph and replayed (the launch-bound
    decode loop without per-call host work): HIP events around the replays, on the stream
    the graph runs on."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            step(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (replays * n)


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_s6(name, one_thread_channels=64):
    """The fp64 oracle, untuned, on the host cores: the whole workload on every thread, and
    a sample of channels of batch row 0 on one thread (the single-core rate)."""
    import numpy as np
    import oracle
    import synth
    inp = synth.workload_inputs(name, seed=(0,))
    d = inp.dims
    nthr = oracle.default_threads()
    elems = d["batch"] * d["L"] * d["d_inner"]
    fn = oracle.s6_grouped_fwd if d.get("ngroups") else oracle.s6_fwd
    reps, t0 = 0, time.perf_counter()
    while True:            # a tiny workload is repeated to about half a second
        fn(**inp.arrays, nthreads=nthr)
        reps += 1
        sec = time.perf_counter() - t0
        if sec > 0.5 or elems * reps > 1e7:
            break
    out = {"value": elems * reps / sec, "unit": "elements/s", "cores": nthr, "kind": "oracle",
           "sample": f"whole {name} workload ({elems} elements x {reps} runs, fp64, {sec:.3f} s wall on "
                     f"{nthr} threads)", "cpu_model": cpu_model()}
    nch = min(one_thread_channels, d["d_inner"])
    units = np.stack([np.zeros(nch, np.int64), np.arange(nch)], 1)
    reps, t0 = 0, time.perf_counter()
    while True:
        fn(**inp.arrays, units=units, nthreads=1)
        reps += 1
        sec1 = time.perf_counter() - t0
        if sec1 > 0.5:
            break
    e1 = nch * d["L"]
    out["value_1thread"] = e1 * reps / sec1
    out["sample_1thread"] = f"{nch} channels of batch row 0 ({e1} elements x {reps} runs, fp64, {sec1:.3f} s, 1 thread)"
    return out


def cpu_baseline_s6_layer(name):
    """The fp64 layer oracle (conv + SiLU, scan, gate), untuned, on the whole workload."""
    import oracle
    import synth
    inp = synth.workload_inputs(name, seed=(0,))
    a, d = inp.arrays, inp.dims
    nthr = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.s6_layer_fwd(a["x"], a["conv_w"], a["conv_b"], a["dt"], a["dt_bias"], a["A_log"], a["B"], a["C"],
                        a["D"], a["h0"], a["conv_state"], a["z"], nthreads=nthr)
    sec = time.perf_counter() - t0
    elems = d["batch"] * d["L"] * d["d_inner"]
    return {"value": elems / sec, "unit": "elements/s", "cores": nthr, "kind": "oracle",
            "sample": f"whole {name} workload ({elems} elements, fp64, {sec:.2f} s wall on {nthr} threads)"}


def cpu_baseline_s6_bwd(name, n_rows=2):
    """The fp64 backward oracle on the first n_rows batch rows of the workload."""
    import oracle
    import synth
    inp = synth.workload_inputs(name, seed=(0,))
    d = inp.dims
    dy, dhf = synth.s6_cotangents(d["batch"], d["L"], d["d_inner"], d["d_state"], seed=(0,))
    nthr = oracle.default_threads()
    n_rows = min(n_rows, d["batch"])
    t0 = time.perf_counter()
    fn = oracle.s6_grouped_bwd if d.get("ngroups") else oracle.s6_bwd
    fn(**inp.arrays, dy=dy, dh_final=dhf, b_range=(0, n_rows), nthreads=nthr)
    sec = time.perf_counter() - t0
    elems = n_rows * d["L"] * d["d_inner"]
    return {"value": elems / sec, "unit": "elements/s", "cores": nthr, "kind": "oracle",
            "sample": f"{n_rows} of {d['batch']} batch rows of the {name} backward "
                      f"({elems} elements, fp64, {sec:.2f} s wall)"}


def cpu_baseline_ssd_bwd(name, n_units=64):
    """The fp64 backward oracle (SSD or trapezoidal) on a bounded sample of (b, head) units,
    with the runner's cotangents."""
    import numpy as np
    import oracle
    import synth
    base = name[: -len("_bwd")]
    inp = synth.workload_inputs(base, seed=(0,))
    d = inp.dims
    w = synth.WORKLOADS[base]
    rng = np.random.default_rng([9 if w["kind"] == "trap" else 5, 0])
    dy = rng.standard_normal((d["batch"], d["L"], d["nheads"], d["headdim"]), dtype=np.float32)
    dhf = rng.standard_normal((d["batch"], d["nheads"], d["headdim"], d["d_state"]), dtype=np.float32)
    nthr = oracle.default_threads()
    n_units = min(n_units, d["batch"] * d["nheads"])
    units = np.stack([np.arange(n_units) % d["batch"], np.arange(n_units) // d["batch"]], 1)
    t0 = time.perf_counter()
    if w["kind"] == "trap":
        oracle.trap_bwd(**inp.arrays, dy=dy, dh_final=dhf, units=units, nthreads=nthr)
    else:
        oracle.ssd_bwd(**inp.arrays, dy=dy, dh_final=dhf, ngroups=d["ngroups"], units=units, nthreads=nthr)
    sec = time.perf_counter() - t0
    elems = n_units * d["L"] * d["headdim"]
    return {"value": elems / sec, "unit": "elements/s", "cores": nthr, "kind": "oracle",
            "sample": f"{n_units} of {d['batch'] * d['nheads']} (b, head) units of the {base} backward "
                      f"({elems} elements, fp64, {sec:.2f} s wall)"}


def ssd_bwd_nseg(d):
    """Segments per (batch, head) the SSD backward uses (mirrors its launch plan)."""
    waves = d["batch"] * d["nheads"] * (d["d_state"] // 32)
    nseg = max(1, min(-(-3072 // waves), d["L"] // 256))
    nseg = max(nseg, -(-d["L"] // 512))
    Ls = -(-(-(-d["L"] // nseg)) // 32) * 32
    return -(-d["L"] // Ls)


def cpu_baseline_units(name, n_units):
    """The fp64 oracle on a bounded sample of (b, h) units of an SSD-type workload."""
    import numpy as np
    import oracle
    import synth
    inp = synth.workload_inputs(name, seed=(0,))
    d = inp.dims
    w = synth.WORKLOADS[name]
    if w["kind"] == "conv":          # one batch row of the conv (numpy oracle)
        a = inp.arrays
        t0 = time.perf_counter()
        oracle.causal_conv1d(a["x"][:1], a["w"], a["bias"], None if a["state"] is None else a["state"][:1],
                             silu=w["silu"])
        sec = time.perf_counter() - t0
        elems = d["L"] * d["channels"]
        return {"value": elems / sec, "unit": "elements/s", "cores": 1, "kind": "oracle",
                "sample": f"1 of {d['batch']} batch rows of {name} ({elems} elements, {sec:.2f} s wall)"}
    nthr = oracle.default_threads()
    total = d["batch"] * d["nheads"]
    n_units = min(n_units, total)
    units = np.stack([np.arange(n_units) % d["batch"], np.arange(n_units) // d["batch"]], 1)
    if w["kind"] == "trap_rot":      # one batch row of the rotation (single-threaded oracle)
        a = inp.arrays
        ang, st = synth.rotation_inputs(1, d["L"], d["nheads"], w["n_angles"])
        t0 = time.perf_counter()
        oracle.trap_rotate(a["k"][:1], a["q"][:1], ang, a["dt"][:1], st)
        sec = time.perf_counter() - t0
        elems = d["L"] * d["nheads"] * d["headdim"]
        return {"value": elems / sec, "unit": "elements/s", "cores": 1, "kind": "oracle",
                "sample": f"1 of {d['batch']} batch rows of {name} ({elems} elements, {sec:.2f} s wall)"}
    def run(units):
        t0 = time.perf_counter()
        if w["kind"] == "trap":
            oracle.trap_fwd(**inp.arrays, units=units, nthreads=nthr)
        elif w["kind"] == "cssd_mimo":
            oracle.cssd_mimo_fwd(**inp.arrays, ngroups=d["ngroups"], units=units, nthreads=nthr)
        else:
            fn = oracle.ssd_fwd if w["kind"] == "ssd" else oracle.cssd_fwd
            fn(**inp.arrays, ngroups=d["ngroups"], units=units, nthreads=nthr)
        return time.perf_counter() - t0

    # a first sample sizes the timed one: as many units as take about CPU_SAMPLE_WALL_S of
    # wall time on the host threads (at most the whole workload)
    sec = run(units)
    n_more = min(total, int(CPU_SAMPLE_WALL_S / max(sec / n_units, 1e-9)))
    if n_more > n_units:
        n_units = n_more
        units = np.stack([np.arange(n_units) % d["batch"], np.arange(n_units) // d["batch"]], 1)
        sec = run(units)
    elems = n_units * d["L"] * d.get("rank", 1) * d["headdim"]
    return {"value": elems / sec, "unit": "elements/s", "cores": nthr, "kind": "oracle",
            "sample": f"{n_units} of {d['batch'] * d['nheads']} (b, head) units of {name} "
                      f"({elems} elements, {sec:.2f} s wall)"}


# the sources each workload's kernels are built from (for the counter-traffic table)
TRAFFIC_SOURCES = {
    "s6": ("device_common.hpp", "s6_kernel.hpp", "s6_scan.hip"),
    "ssd": ("device_common.hpp", "ssd_scan.hip"),
    "cssd": ("device_common.hpp", "cssd_scan.hip"),
}


def src_sha1(kind):
    import hashlib
    h = hashlib.sha1()
    for f in TRAFFIC_SOURCES.get(kind, ()):
        h.update(open(os.path.join(ROOT, "selective_state_space_s6_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def counter_traffic(name, kind):
    """Counter-measured HBM bytes per call, or None if the kernels changed since."""
    ent = TRAFFIC.get(name)
    if ent is None or kind not in TRAFFIC_SOURCES or src_sha1(kind) != ent["src_sha1"]:
        return None
    return round(ent["bytes"])


def measure(name, dev, steps, warmup):
    step, dims, w, kernels = make_runner(name, dev)
    wall, per = time_steps(step, steps, warmup)
    graph_us = graph_us_per_step(step) if dims.get("L") == 1 else None
    ms = wall * 1e3 / steps
    kind = w["kind"]
    dims = dict(dims, chunk_len=w.get("chunk_len"))
    if w.get("carry"):
        dims["carry"] = True
    if kind == "copy":
        elems, bytes_, ops = dims["bytes"] // 8, dims["bytes"], 0
    elif kind == "s6":
        elems, bytes_, ops = s6_model(dims)
    elif kind == "s6_layer":
        elems, bytes_, ops = s6_layer_model(dims)
    elif kind == "s6_pc":
        elems, bytes_, ops = s6_pc_model(dims)
    elif kind in ("s6_save", "s6_pc_save"):      # the forward plus the saved states it writes
        elems, bytes_, ops = s6_model(dims) if kind == "s6_save" else s6_pc_model(dims)
        bytes_ += dims["batch"] * (-(-dims["L"] // 16)) * dims["d_inner"] * dims["d_state"] * 4
    elif kind == "s6_bwd":
        elems, bytes_, ops = s6_bwd_model(dims)
    elif kind == "ssd_bwd":
        elems, bytes_, ops = ssd_bwd_model(dict(dims, nseg=ssd_bwd_nseg(dims)))
    elif kind == "trap_bwd":       # the SSD backward with one group per head, plus the q.k pass
        dd = dict(dims, ngroups=dims["nheads"])
        elems, bytes_, ops = ssd_bwd_model(dict(dd, nseg=ssd_bwd_nseg(dd)))
    elif kind == "ssd":
        elems, bytes_, ops = ssd_model(dims)
    elif kind == "trap":
        elems, bytes_, ops = trap_model(dims)
    elif kind == "trap_rot":
        elems, bytes_, ops = trap_rot_model(dims)
    elif kind == "conv":
        elems, bytes_, ops = conv_model(dims)
    elif kind == "cssd_mimo":
        elems, bytes_, ops = mimo_model(dims)
    else:
        elems, bytes_, ops = cssd_model(dims)
    ev_ms = sorted(per)[len(per) // 2]
    return dict(name=name, kind=kind, dims=dims, dtype=w["dtype"], ms=ms, event_ms_median=ev_ms,
                event_ms=per, elems=elems, bytes=bytes_, ops=ops, kernels=kernels, graph_us=graph_us)


HEADLINE = "ssd_long"
# the five workloads of the scope, in order: S6 tiny, S6 Mamba-1 layer, SSD Mamba-2 layer,
# long-context SSD, complex SSD
CONFIGS = ("s6_tiny", "s6_mamba1", "ssd_mamba2", "ssd_long", "cssd_mamba3")
SECONDARY = (("s6_long", 10), ("s6_long_walk", 5), ("cssd_mimo_mamba3", 5), ("s6_pc_mamba1", 10),
             ("trap_mamba3", 5), ("trap_rot_mamba3", 5), ("conv_mamba2", 10), ("s6_layer_mamba1", 10),
             ("s6_decode_mamba1", 50), ("ssd_decode_mamba2", 50), ("trap_decode_mamba3", 50),
             ("s6_mamba1_bwd", 10), ("s6_mamba1_fwd_save", 10), ("s6_mamba1_bwd_saved", 10),
             ("s6_pc_mamba1_fwd_save", 5), ("s6_pc_mamba1_bwd_saved", 5), ("s6_pc_mamba1_bwd", 5),
             ("ssd_mamba2_bwd", 5), ("trap_mamba3_bwd", 5))


def roofline(m):
    """The roofline object of one measured workload: the bound its path is priced on, the
    achieved rate from the algorithmic bytes or flops of a call over the call's HIP-event
    time (median), the counter traffic when it is current, and labelled extra fractions."""
    kind, name = m["kind"], m["name"]
    ev_s = m["event_ms_median"] * 1e-3
    gbs = m["bytes"] / ev_s / 1e9
    kern = {"kernel": " + ".join(m["kernels"]), "kernel_ms": round(m["event_ms_median"], 5)}
    if kind == "s6":
        # priced on HBM; the issue-slot fraction of the instruction mix is an extra field
        updates = m["elems"] * m["dims"]["d_state"]
        slots_frac = updates * S6_SLOTS_PER_UPDATE / ev_s / VALU_SLOTS_PER_S
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": counter_traffic(name, "s6"),
                "algorithmic_bytes": m["bytes"], **kern,
                "issue_slot_frac": round(slots_frac, 4),
                "issue_slot_basis": f"{S6_SLOTS_PER_UPDATE} fp32 VALU issue slots per state update (exact "
                                    "hold incl.), 39.3 T lane-slots/s (256 CU x 4 SIMD x 16 lanes x 2.4 GHz)"}
    if kind in ("ssd", "trap") and m["dims"].get("L", 2) > 1:
        # below the bf16 ridge (~165 flop/B against ~315): priced on HBM, with the
        # matrix-core fraction of the method's flops (the target metric) alongside
        tf = m["ops"] / ev_s / 1e12
        pk, basis = MFMA_PEAKS[kind]
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": counter_traffic(name, "ssd"),
                "algorithmic_bytes": m["bytes"], **kern,
                "mfma_TFLOPs": round(tf, 2), "mfma_peak": pk, "mfma_frac": round(tf / pk, 4),
                "algorithmic_flops": m["ops"], "mfma_basis": basis}
    if kind in MFMA_PEAKS and m["dims"].get("L", 2) > 1:
        tf = m["ops"] / ev_s / 1e12
        pk, basis = MFMA_PEAKS[kind]
        tr_kind = "cssd" if kind in ("cssd", "cssd_mimo") else None
        return {"bound": "mfma", "achieved": round(tf, 2), "peak": pk, "unit": "TFLOP/s",
                "frac": round(tf / pk, 4), "traffic": counter_traffic(name, tr_kind) if tr_kind else None,
                "algorithmic_flops": m["ops"], "peak_basis": basis, **kern,
                "hbm_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": m["bytes"]}
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": m["bytes"], **kern}


def cpu_baseline(name, kind):
    if kind in ("s6", "s6_pc", "s6_save", "s6_pc_save"):
        return cpu_baseline_s6(name)
    if kind == "s6_bwd":
        return cpu_baseline_s6_bwd(name)
    if kind == "s6_layer":
        return cpu_baseline_s6_layer(name)
    if kind in ("ssd_bwd", "trap_bwd"):
        return cpu_baseline_ssd_bwd(name)
    out = cpu_baseline_units(name, 16)
    out["cpu_model"] = cpu_model()
    return out


def dtype_of(m):
    return {"s6": "f32", "cssd": "f32"}.get(m["kind"], "bf16" if m["dtype"] == "bf16" else "f32")


def config_line(m):
    return {"workload": m["name"], "value": round(m["elems"] / (m["ms"] * 1e-3), 1), "unit": "elements/s",
            "ms_per_step": round(m["ms"], 5), "dtype": dtype_of(m),
            "config": {k: v for k, v in m["dims"].items() if v is not None}, "roofline": roofline(m)}


def secondary_line(s):
    es = s["event_ms_median"] * 1e-3
    ent = {"workload": s["name"], "value": round(s["elems"] / (s["ms"] * 1e-3), 1), "unit": "elements/s",
           "ms_per_step": round(s["ms"], 4), "kernel_ms": round(s["event_ms_median"], 4),
           "hbm_GBps": round(s["bytes"] / es / 1e9, 1), "hbm_frac": round(s["bytes"] / es / 1e9 / HBM_PEAK_GBS, 4)}
    if s["kind"] in ("s6", "s6_layer", "s6_pc", "s6_save", "s6_pc_save"):
        upd = s["elems"] * s["dims"]["d_state"]
        ent["issue_slot_frac"] = round(upd * S6_SLOTS_PER_UPDATE / es / VALU_SLOTS_PER_S, 4)
        if s["dims"].get("segmented"):
            ent["segmented"] = True
        if s["dims"]["L"] == 1:
            ent["us_per_step_eager"] = round(s["event_ms_median"] * 1e3, 2)
            ent["us_per_step_graph"] = round(s["graph_us"], 2)
    elif s["kind"] == "s6_bwd":
        ent["fp32_TFLOPs"] = round(s["ops"] / es / 1e12, 2)
    elif s["kind"] in ("ssd_bwd", "trap_bwd"):
        ent["mfma_fp32_TFLOPs"] = round(s["ops"] / es / 1e12, 2)
        ent["mfma_frac_fp32"] = round(s["ops"] / es / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)
        ent["mfma_basis"] = "executed 16x16x4 fp32 MFMAs of the walks"
    elif s["kind"] in ("cssd", "cssd_mimo"):
        ent["mfma_fp32_TFLOPs"] = round(s["ops"] / es / 1e12, 2)
        ent["mfma_frac_fp32"] = round(s["ops"] / es / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)
    elif s["kind"] in ("ssd", "trap") and s["dims"]["L"] == 1:
        ent["us_per_step_eager"] = round(s["event_ms_median"] * 1e3, 2)
        ent["us_per_step_graph"] = round(s["graph_us"], 2)
    elif s["kind"] in ("ssd", "trap"):
        ent["mfma_TFLOPs"] = round(s["ops"] / es / 1e12, 1)
        ent["mfma_frac_bf16"] = round(s["ops"] / es / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
    return ent


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="measure this workload alone (headline schema)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copies", type=int, default=N_ROTATE, help="input copies rotated between steps")
    args = ap.parse_args()
    globals()["N_ROTATE"] = max(1, args.copies)
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); the scan "
              "shards over batch and heads with no communication, and no multi-GPU path exists here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")

    single = args.workload is not None
    head = args.workload or HEADLINE
    log(f"[bench] headline {head}: warmup {args.warmup}, steps {args.steps}")
    m = measure(head, dev, args.steps, args.warmup)
    if m["kind"] == "copy":
        gbs = m["bytes"] / (m["event_ms_median"] * 1e-3) / 1e9
        print(json.dumps({"workload": "copy_1gib", "bytes_per_call": m["bytes"], "event_ms_median":
                          round(m["event_ms_median"], 5), "GBps": round(gbs, 1)}), flush=True)
        return
    line = config_line(m)
    out = {
        "metric": "scan elements/s (batch*L*d_inner)",
        "value": line["value"],
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": line["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": line["dtype"],
        "data": "synthetic",
        "config": {"workload": head, **line["config"]},
        "roofline": line["roofline"],
    }
    # every GPU measurement first, then the host-side oracle baselines, so that no
    # measurement follows a stretch of host work with the GPU idle
    kinds = {head: m["kind"]}
    del m
    torch.cuda.empty_cache()
    if not single:
        cfgs = []
        for name in CONFIGS:
            if name == head:
                c = dict(line)
            else:
                log(f"[bench] config {name}")
                cm = measure(name, dev, args.steps, args.warmup)
                c = config_line(cm)
                kinds[name] = cm["kind"]
                del cm
                torch.cuda.empty_cache()
            cfgs.append(c)
        out["configs"] = cfgs
    if not single and not args.no_secondary:
        sec = []
        for name, steps in SECONDARY:
            log(f"[bench] secondary {name}")
            s = measure(name, dev, steps, 2)
            sec.append(secondary_line(s))
            del s
            torch.cuda.empty_cache()
        out["secondary"] = sec
    if not args.no_cpu:
        log(f"[bench] cpu baseline (oracle) {head}")
        out["cpu_baseline"] = cpu_baseline(head, kinds[head])
        for c in out.get("configs", []):
            name = c["workload"]
            if name == head:
                c["cpu_baseline"] = out["cpu_baseline"]
            else:
                log(f"[bench] cpu baseline (oracle) {name}")
                c["cpu_baseline"] = cpu_baseline(name, kinds[name])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
