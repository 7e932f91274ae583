"""HIP graph capture of the chunked and backward entry points: the library allocates,
clears and synchronises nothing inside a call, so one call captured into a graph and replayed
gives the eager call's outputs bit for bit.  Each replay follows eager work that poisons the
outputs (NaN fill) and a synchronisation."""
import pytest
import torch

import synth
from helpers import lib

pytestmark = pytest.mark.gpu


def _capture_and_replay(fn, outs):
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r)


def test_capture_s6_and_saved_pair(cuda_device):
    m = lib()
    inp = synth.s6_inputs(2, 300, 64, 16, seed=(81,), h0=True)
    t = inp.torch(cuda_device)
    y = torch.empty(2, 300, 64, device=cuda_device)
    hf = torch.empty(2, 64, 16, device=cuda_device)
    ck = torch.empty(2, 19, 64, 16, device=cuda_device)
    dy = torch.randn(2, 300, 64, device=cuda_device)
    shapes = dict(du=(2, 300, 64), ddt=(2, 300, 64), dB=(2, 300, 16), dC=(2, 300, 16), dA_log=(64, 16),
                  dD=(64,), ddt_bias=(64,), dh0=(2, 64, 16))
    out = {k: torch.empty(v, device=cuda_device) for k, v in shapes.items()}
    ws = torch.empty(m.ssm_s6_scan_bwd_workspace_size(2, 300, 64, 16), dtype=torch.uint8, device=cuda_device)

    def fwd():
        m.ssm_s6_scan_fwd(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"], y=y,
                          h_final=hf)
    _capture_and_replay(fwd, [y, hf])

    def pair():
        m.ssm_s6_scan_fwd_save(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"], y=y,
                               h_final=hf, checkpoints=ck)
        m.ssm_s6_scan_bwd_saved(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"], dy,
                                None, ck, out=out, workspace=ws)
    _capture_and_replay(pair, [y, hf, ck, *out.values()])


def test_capture_ssd_forward_and_backward(cuda_device):
    m = lib()
    inp = synth.ssd_inputs(1, 1100, 2, 64, 128, 1, seed=(82,), dtype="bf16", h0=True)
    t = inp.torch(cuda_device)
    y = torch.empty(1, 1100, 2, 64, device=cuda_device)
    hf = torch.empty(1, 2, 64, 128, device=cuda_device)
    wsf = torch.empty(max(1, m.ssd_chunk_scan_fwd_workspace_size(1, 1100, 2, 64, 128, 1, 256)), dtype=torch.uint8,
                      device=cuda_device)

    def fwd():
        m.ssd_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                             chunk_len=256, y=y, h_final=hf, workspace=wsf)
    _capture_and_replay(fwd, [y, hf])

    dy = torch.randn(1, 1100, 2, 64, device=cuda_device)
    dhf = torch.randn(1, 2, 64, 128, device=cuda_device)
    wsb = torch.empty(m.ssd_chunk_scan_bwd_workspace_size(1, 1100, 2, 64, 128, 1, 256), dtype=torch.uint8,
                      device=cuda_device)
    out = {}

    def bwd():
        g = m.ssd_chunk_scan_bwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"], dy,
                                 dhf, chunk_len=256, out=out or None, workspace=wsb)
        out.update({k: v for k, v in g.items() if v is not None})
    bwd()
    _capture_and_replay(bwd, list(out.values()))


def test_capture_trap_backward(cuda_device):
    m = lib()
    inp = synth.trap_inputs(1, 700, 2, 64, 128, seed=(83,), h0=True, prev=True)
    t = inp.torch(cuda_device)
    dy = torch.randn(1, 700, 2, 64, device=cuda_device)
    dhf = torch.randn(1, 2, 64, 128, device=cuda_device)
    ws = torch.empty(m.ssd_trap_chunk_scan_bwd_workspace_size(1, 700, 2, 64, 128, 64), dtype=torch.uint8,
                     device=cuda_device)
    out = {}

    def bwd():
        g = m.ssd_trap_chunk_scan_bwd(t["x"], t["k"], t["q"], t["dt"], t["a"], t["trap"], t["D"], t["h0"],
                                      t["k_prev"], t["x_prev"], dy, dhf, out=out or None, workspace=ws)
        out.update({k: v for k, v in g.items() if v is not None})
    bwd()
    _capture_and_replay(bwd, list(out.values()))


def test_capture_cssd_mimo(cuda_device):
    m = lib()
    inp = synth.mimo_inputs(1, 300, 4, 2, 64, 32, seed=(84,), h0=True)
    t = inp.torch(cuda_device)
    y = torch.empty(1, 300, 4, 2, 64, device=cuda_device)
    hf = torch.empty(1, 2, 64, 32, 2, device=cuda_device)
    ws = torch.empty(max(1, m.ssd_cplx_mimo_chunk_scan_fwd_workspace_size(1, 300, 4, 2, 64, 32, 1, 64)),
                     dtype=torch.uint8, device=cuda_device)

    def fwd():
        m.ssd_cplx_mimo_chunk_scan_fwd(t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                       y=y, h_final=hf, workspace=ws)
    _capture_and_replay(fwd, [y, hf])


def test_capture_grouped_saved_pair(cuda_device):
    m = lib()
    inp = synth.s6_inputs(2, 200, 48, 16, seed=(85,), h0=True, ngroups=48)
    t = inp.torch(cuda_device)
    y = torch.empty(2, 200, 48, device=cuda_device)
    hf = torch.empty(2, 48, 16, device=cuda_device)
    ck = torch.empty(2, 13, 48, 16, device=cuda_device)
    dy = torch.randn(2, 200, 48, device=cuda_device)
    shapes = dict(du=(2, 200, 48), ddt=(2, 200, 48), dB=(2, 200, 48, 16), dC=(2, 200, 48, 16), dA_log=(48, 16),
                  dD=(48,), ddt_bias=(48,), dh0=(2, 48, 16))
    out = {k: torch.empty(v, device=cuda_device) for k, v in shapes.items()}
    ws = torch.empty(m.ssm_s6_scan_grouped_bwd_workspace_size(2, 200, 48, 16, 48), dtype=torch.uint8,
                     device=cuda_device)

    def pair():
        m.ssm_s6_scan_grouped_fwd_save(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                       y=y, h_final=hf, checkpoints=ck)
        m.ssm_s6_scan_grouped_bwd_saved(t["u"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"],
                                        dy, None, ck, out=out, workspace=ws)
    _capture_and_replay(pair, [y, hf, ck, *out.values()])
