"""GPU parity of the convolution's gradients (eqtp_conv_backward, through the
C ABI) against the fp64 oracle's gradients on the same seeded inputs.

Bar: max|gpu - oracle| <= 2e-4 * max|oracle| per gradient tensor (grad_x,
grad_w, grad_vec), as for the forward.
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _say, _t

pytestmark = pytest.mark.gpu


def _gout(wl, seed):
    K = (wl.lmax + 1) ** 2
    return np.random.default_rng(seed).standard_normal((wl.N, wl.C, K)).astype(np.float32)


def _check(eq, wl, gout, unsorted=False, perm_seed=2026, need=(True, True, True), what=""):
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, wl.lmax, wl.path_set)
    if unsorted:
        rng = np.random.default_rng(perm_seed)
        perm = rng.permutation(wl.src.shape[0])
        vec, src, dst = wl.vec[perm], wl.src[perm], wl.dst[perm]
        gx, gw, gv = eq.eqtp_conv_backward(_t(vec), _t(src), _t(wl.x), _t(wl.w), _t(gout), wl.lmax, dst=_t(dst),
                                           path_set=wl.path_set, need_x=need[0], need_w=need[1], need_vec=need[2])
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.shape[0])
        gv_np = _np(gv)[inv] if gv is not None else None
    else:
        gx, gw, gv = eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), _t(gout), wl.lmax,
                                           row_ptr=_t(wl.row_ptr), path_set=wl.path_set, need_x=need[0],
                                           need_w=need[1], need_vec=need[2])
        gv_np = _np(gv) if gv is not None else None
    for got, r, name, want in ((gx, ref[0], "grad_x", need[0]), (gw, ref[1], "grad_w", need[1]),
                               (gv_np, ref[2], "grad_vec", need[2])):
        if not want:
            assert got is None
            continue
        got = got if isinstance(got, np.ndarray) else _np(got)
        _assert_close(got, r, TOL, what + " " + name)


@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", [0, 1])
@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
def test_backward_small_sorted(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(37, 9, C, lmax, 300 + lmax * 10 + C, path_set=ps, empty_rows=(3,), long_rows=(5,),
                           long_len=70, zero_vec_edges=1)
    _say("backward sorted lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.src.shape[0]))
    _check(eq, wl, _gout(wl, 7), what="sorted L%d ps%d C%d" % (lmax, ps, C))


@pytest.mark.parametrize("lmax,ps,C", [(3, 0, 64), (3, 1, 32), (2, 0, 8), (1, 0, 128), (3, 0, 128)])
def test_backward_small_unsorted(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(41, 10, C, lmax, 500 + lmax + C, path_set=ps, empty_rows=(0,), zero_vec_edges=2)
    _say("backward unsorted lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.src.shape[0]))
    _check(eq, wl, _gout(wl, 8), unsorted=True, what="unsorted L%d ps%d C%d" % (lmax, ps, C))


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True),
                                  (True, False, True)])
def test_backward_partial_requests(need):
    eq = _eq()
    wl = synth.small_graph(23, 8, 32, 3, 77)
    _say("backward partial %s" % (need,))
    _check(eq, wl, _gout(wl, 9), need=need, what="partial")


def test_backward_typical_workload():
    eq = _eq()
    wl = synth.make_config("typical")
    _say("backward typical E=%d" % wl.src.shape[0])
    _check(eq, wl, _gout(wl, 10), what="typical")


def test_backward_zero_length_edges_give_zero_grad_vec():
    eq = _eq()
    wl = synth.small_graph(12, 6, 16, 3, 88, zero_vec_edges=4)
    _say("backward zero-length edges")
    _, _, gv = eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), _t(_gout(wl, 11)), 3,
                                     row_ptr=_t(wl.row_ptr))
    assert np.all(_np(gv)[:4] == 0.0)


def test_backward_no_edges():
    eq = _eq()
    import torch

    N, C = 5, 16
    x = torch.randn(N, C, 16, device="cuda")
    w = torch.randn(23, C, device="cuda")
    g = torch.randn(N, C, 16, device="cuda")
    rp = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    vec = torch.zeros(0, 3, device="cuda")
    src = torch.zeros(0, dtype=torch.int32, device="cuda")
    _say("backward no edges")
    gx, gw, gv = eq.eqtp_conv_backward(vec, src, x, w, g, 3, row_ptr=rp)
    assert float(_np(gx).__abs__().max()) == 0.0 and float(_np(gw).__abs__().max()) == 0.0
    assert gv.shape == (0, 3)


def test_autograd_function_matches_backward_and_oracle():
    import torch

    eq = _eq()
    from spherical_harmonic_cg_amd.autograd import equivariant_conv

    wl = synth.small_graph(19, 7, 32, 3, 99, zero_vec_edges=1)
    gout = _gout(wl, 12)
    vec = _t(wl.vec).requires_grad_(True)
    x = _t(wl.x).requires_grad_(True)
    w = _t(wl.w).requires_grad_(True)
    _say("autograd function")
    out = equivariant_conv(vec, x, w, _t(wl.src), 3, row_ptr=_t(wl.row_ptr))
    ref_out = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, 3)
    _assert_close(_np(out.detach()), ref_out, TOL, "autograd forward")
    (out * _t(gout)).sum().backward()
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, 3)
    _assert_close(_np(x.grad), ref[0], TOL, "autograd grad_x")
    _assert_close(_np(w.grad), ref[1], TOL, "autograd grad_w")
    _assert_close(_np(vec.grad), ref[2], TOL, "autograd grad_vec")
    # only the edge vectors (forces)
    vec2 = _t(wl.vec).requires_grad_(True)
    out2 = equivariant_conv(vec2, _t(wl.x), _t(wl.w), _t(wl.src), 3, row_ptr=_t(wl.row_ptr))
    (out2 * _t(gout)).sum().backward()
    _assert_close(_np(vec2.grad), ref[2], TOL, "autograd grad_vec only")
