"""GPU parity of the interaction layer (eqtp_interaction, through the C ABI)
against the fp64 oracle's layer (oracle_interaction) on the same seeded
inputs: channel linear, radial network (SiLU), convolution with the network's
per-edge path weights (last layer on the matrix cores), channel linear, 1/norm.

Bar: max|gpu - oracle| <= 2e-4 * max|oracle| over the whole output.
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _say, _t

pytestmark = pytest.mark.gpu


def _run(eq, wl, iw, norm, workspace=None):
    return eq.eqtp_interaction(_t(wl.vec), _t(wl.src), _t(wl.row_ptr), _t(wl.x), _t(iw.W_up), _t(iw.W1), _t(iw.W2),
                               _t(iw.W3), _t(iw.W_out), wl.lmax, wl.r_cut, norm=norm, path_set=wl.path_set,
                               workspace=workspace)


def _ref(wl, iw, norm):
    return oracle.interaction(wl.N, wl.vec, wl.src, wl.dst, wl.x, iw.W_up, iw.W1, iw.W2, iw.W3, iw.W_out, wl.lmax,
                              wl.r_cut, norm=norm, path_set=wl.path_set)


@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", [0, 1])
@pytest.mark.parametrize("C", [16, 64, 128])
def test_interaction_small(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(35, 9, C, lmax, 1200 + 10 * lmax + C + ps, path_set=ps, radial=True, r_cut=5.0,
                           empty_rows=(2,), long_rows=(4,), long_len=45, zero_vec_edges=1)
    iw = synth.interaction_weights(lmax, C, ps, seed=1300 + lmax + C)
    _say("interaction small lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.src.shape[0]))
    _assert_close(_np(_run(eq, wl, iw, 3.0)), _ref(wl, iw, 3.0), TOL, "interaction L%d ps%d C%d" % (lmax, ps, C))


def test_interaction_edges_beyond_cutoff_and_no_edges():
    eq = _eq()
    wl = synth.small_graph(20, 7, 32, 3, 1401, radial=True, r_cut=5.0)
    iw = synth.interaction_weights(3, 32, 0, seed=1401)
    far = wl.vec / np.linalg.norm(wl.vec, axis=1, keepdims=True) * 6.0
    wl.vec[::3] = far[::3].astype(np.float32)  # every third edge past the cut-off: no weight
    _say("interaction cut-off E=%d" % wl.src.shape[0])
    _assert_close(_np(_run(eq, wl, iw, 1.0)), _ref(wl, iw, 1.0), TOL, "interaction cut-off")
    empty = synth.small_graph(5, 0, 32, 3, 1402, radial=True, r_cut=5.0, empty_rows=range(5))
    out = _np(_run(eq, empty, iw, 1.0))
    assert np.all(out == 0.0)


def test_interaction_workspace_reuse():
    """Two calls on one caller-given workspace (the second smaller) match their own oracles."""
    eq = _eq()
    import torch

    a = synth.small_graph(60, 12, 64, 3, 1403, radial=True, r_cut=5.0)
    b = synth.small_graph(17, 5, 64, 3, 1404, radial=True, r_cut=5.0)
    iw = synth.interaction_weights(3, 64, 0, seed=1403)
    n = eq.eqtp_interaction_workspace_bytes(a.N, a.src.shape[0], 3, 64)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    _say("interaction workspace reuse")
    _assert_close(_np(_run(eq, a, iw, 2.0, workspace=ws)), _ref(a, iw, 2.0), TOL, "first call")
    _assert_close(_np(_run(eq, b, iw, 2.0, workspace=ws)), _ref(b, iw, 2.0), TOL, "second call")


def test_interaction_mid_workload_full():
    """The mid graph (10k atoms, r_c = 4 A, 266k edges, L = 3, C = 64) through one interaction layer
    (H = 64, norm = mean degree): every output entry against the oracle."""
    eq = _eq()
    wl = synth.make_config("mid")
    iw = synth.interaction_weights(3, 64, 0)
    norm = wl.src.shape[0] / wl.N
    _say("interaction mid E=%d" % wl.src.shape[0])
    err = _assert_close(_np(_run(eq, wl, iw, norm)), _ref(wl, iw, norm), TOL, "interaction mid")
    _say("interaction mid rel error %.2e" % err)
