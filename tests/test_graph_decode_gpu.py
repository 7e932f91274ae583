"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph on ROCm): the launch-bound
serving loop.  Eight L = 1 steps carrying the state in place are captured once; each replay
starts from the same entering state (restored eagerly between replays, with a device
synchronisation) and must equal the eager chain bit for bit, on every replay.  The library
records no memset or allocation; the outputs are preallocated."""
import pytest

import synth
from helpers import lib

pytestmark = pytest.mark.gpu

T = 8
REPLAYS = 3


def _replay_check(step_fn, state_tensors, out_tensors, device):
    import torch
    init = [s.clone() for s in state_tensors]
    # eager reference
    for s in range(T):
        step_fn(s)
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in out_tensors]
    ref_state = [s.clone() for s in state_tensors]
    # capture (from the initial state; warm the allocator and kernels up on a side stream first)
    for s_, i_ in zip(state_tensors, init):
        s_.copy_(i_)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(T):
            step_fn(s)
    torch.cuda.synchronize()
    for _ in range(REPLAYS):
        for s_, i_ in zip(state_tensors, init):
            s_.copy_(i_)
        for o in out_tensors:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(out_tensors, ref_out):
            assert torch.equal(o, r)
        for s_, r in zip(state_tensors, ref_state):
            assert torch.equal(s_, r)


def test_graph_s6_fused_decode(cuda_device):
    import torch
    inp = synth.layer_inputs(16, T, 256, 16, 4, seed=(91,), h0=True)
    t = inp.torch(cuda_device)
    h, st = t["h0"].clone(), t["conv_state"].clone()
    ys = [torch.empty((16, 1, 256), dtype=torch.float32, device=cuda_device) for _ in range(T)]
    sl = [{n: t[n][:, s:s + 1].clone() for n in ("x", "dt", "B", "C", "z")} for s in range(T)]
    m = lib()

    def step(s):
        m.ssm_s6_fused_fwd(sl[s]["x"], t["conv_w"], t["conv_b"], sl[s]["dt"], t["dt_bias"], t["A_log"],
                           sl[s]["B"], sl[s]["C"], t["D"], h, st, sl[s]["z"], y=ys[s], h_final=h,
                           conv_state_out=st)
    _replay_check(step, [h, st], ys, cuda_device)


def test_graph_ssd_and_trap_decode(cuda_device):
    import torch
    m = lib()
    inp = synth.ssd_inputs(8, T, 4, 64, 128, 1, seed=(92,), h0=True, D="normal")
    t = inp.torch(cuda_device)
    h = t["h0"].clone()
    ys = [torch.empty((8, 1, 4, 64), dtype=torch.float32, device=cuda_device) for _ in range(T)]
    ws = torch.empty((max(1, m.ssd_chunk_scan_fwd_workspace_size(8, 1, 4, 64, 128, 1, 256)),), dtype=torch.uint8,
                     device=cuda_device)
    sl = [{n: t[n][:, s:s + 1].clone() for n in ("x", "dt", "B", "C")} for s in range(T)]

    def step(s):
        m.ssd_chunk_scan_fwd(sl[s]["x"], sl[s]["dt"], t["dt_bias"], t["A_log"], sl[s]["B"], sl[s]["C"], t["D"], h,
                             y=ys[s], h_final=h, workspace=ws)
    _replay_check(step, [h], ys, cuda_device)

    inp = synth.trap_inputs(8, T, 4, 64, 128, seed=(93,), h0=True, prev=True)
    t = inp.torch(cuda_device)
    h2 = t["h0"].clone()
    y2 = [torch.empty((8, 1, 4, 64), dtype=torch.float32, device=cuda_device) for _ in range(T)]
    ws2 = torch.empty((m.ssd_trap_chunk_scan_fwd_workspace_size(8, 1, 4, 64, 128, 64),), dtype=torch.uint8,
                      device=cuda_device)
    sl2 = [{n: t[n][:, s:s + 1].clone() for n in ("x", "k", "q", "dt", "a", "trap")} for s in range(T)]
    prev = [(t["k_prev"], t["x_prev"])] + [(sl2[s]["k"][:, 0].clone(), sl2[s]["x"][:, 0].clone()) for s in range(T - 1)]

    def step2(s):
        m.ssd_trap_chunk_scan_fwd(sl2[s]["x"], sl2[s]["k"], sl2[s]["q"], sl2[s]["dt"], sl2[s]["a"], sl2[s]["trap"],
                                  t["D"], h2, prev[s][0], prev[s][1], y=y2[s], h_final=h2, workspace=ws2)
    _replay_check(step2, [h2], y2, cuda_device)
