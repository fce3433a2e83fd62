"""A fused convolution + channel linear captured once as a HIP graph (through
torch.cuda.CUDAGraph) and replayed: every replay must reproduce the eager
result bit for bit (dst-sorted edges are deterministic), with eager work on
the same buffers between the replays."""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth

pytestmark = pytest.mark.gpu


def test_conv_linear_graph_replay():
    import torch

    import spherical_harmonic_cg_amd as eq

    eq.load_library()
    dev = torch.device("cuda:0")
    wl = synth.small_graph(n=300, e_per_row=21, C=64, lmax=3, seed=77, empty_rows=(5,), long_rows=(9,),
                           long_len=90)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    vec, src, rp, x, w, wlin = T(wl.vec), T(wl.src), T(wl.row_ptr), T(wl.x), T(wl.w), T(wl.w_lin)
    out = torch.empty((wl.N, wl.C, wl.K), dtype=torch.float32, device=dev)
    h = torch.empty_like(out)

    def step():
        eq.eqtp_conv_fused(vec, src, x, w, 3, row_ptr=rp, out=out)
        eq.eqtp_linear(out, wlin, 3, eq.EQTP_BF16, out=h)

    step()
    torch.cuda.synchronize()
    ref_out, ref_h = out.clone(), h.clone()
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, 3)
    err = np.abs(ref_out.cpu().numpy() - ref).max() / np.abs(ref).max()
    assert err <= 2e-4

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        h.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "replay %d: conv differs from the eager result" % r
        assert torch.equal(h, ref_h), "replay %d: linear differs from the eager result" % r
        step()  # eager work on the same buffers between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
