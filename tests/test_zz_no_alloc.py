"""GPU check of ssd_chunk_scan_fwd_noalloc (the SSD forward whose segment states live in the
library's static device scratch) against ssd_chunk_scan_fwd with a caller workspace: the
same kernels, so the outputs must be bitwise equal; two calls in a row, the second with a
smaller input, and both against the fp64 oracle at the bf16 bar."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL_BF16, lib, report

pytestmark = pytest.mark.gpu

DT = oracle.BBAR_DT

SHAPES = [  # batch, L, nheads, headdim, d_state, ngroups: long enough for several segments
    (2, 3000, 4, 64, 128, 2),
    (1, 1200, 3, 64, 64, 1),      # smaller: fewer segments, smaller states than the first call
]


def test_noalloc_equals_workspace_entry(cuda_device):
    m = lib()
    for i, (batch, L, H, P, N, G) in enumerate(SHAPES):
        assert m.ssd_chunk_scan_fwd_workspace_size(batch, L, H, P, N, G, 256) > 0   # segments in use
        inp = synth.ssd_inputs(batch, L, H, P, N, G, seed=(90, i), h0=True)
        t = inp.torch(cuda_device)
        args = (t["x"], t["dt"], t["dt_bias"], t["A_log"], t["B"], t["C"], t["D"], t["h0"])
        y_ws, h_ws = m.ssd_chunk_scan_fwd(*args, chunk_len=256, flags=DT, return_final=True)
        y_na = torch.empty_like(y_ws)
        h_na = torch.empty_like(h_ws)
        m.ssd_chunk_scan_fwd_noalloc(*args, chunk_len=256, flags=DT, y=y_na, h_final=h_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws) and torch.equal(h_na, h_ws), (batch, L, H, P, N, G)
        yo, ho = oracle.ssd_fwd(**inp.arrays, ngroups=G, flags=DT)
        ey = synth.max_rel_err(y_na.cpu().numpy(), yo)
        eh = synth.max_rel_err(h_na.cpu().numpy(), ho)
        report(f"ssd noalloc {(batch, L, H, P, N, G)}", y=ey, h_final=eh)
        assert ey <= TOL_BF16 and eh <= TOL_BF16
