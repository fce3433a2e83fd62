"""GPU parity of the gradients of the radial-weight convolution
(eqtp_conv_backward with EQTP_W_RADIAL, through the C ABI) against the fp64
oracle's gradients (oracle_conv_backward_radial) on the same seeded inputs.

Bar: max|gpu - oracle| <= 2e-4 * max|oracle| per gradient tensor (grad_x,
grad_W, grad_vec), as for the forward.  All three are sums of fp32 atomics
on the GPU (grad_vec over the 16-channel blocks).
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _say, _t

pytestmark = pytest.mark.gpu

RAD = 1  # EQTP_W_RADIAL


def _gout(wl, seed):
    K = (wl.lmax + 1) ** 2
    return np.random.default_rng(seed).standard_normal((wl.N, wl.C, K)).astype(np.float32)


def _run(eq, wl, vec, src, dst, gout, unsorted, need):
    if unsorted:
        return eq.eqtp_conv_backward(_t(vec), _t(src), _t(wl.x), _t(wl.w_rad), _t(gout), wl.lmax, dst=_t(dst),
                                     path_set=wl.path_set, need_x=need[0], need_w=need[1], need_vec=need[2],
                                     weight_mode=RAD, r_cut=wl.r_cut)
    return eq.eqtp_conv_backward(_t(vec), _t(src), _t(wl.x), _t(wl.w_rad), _t(gout), wl.lmax,
                                 row_ptr=_t(wl.row_ptr), path_set=wl.path_set, need_x=need[0], need_w=need[1],
                                 need_vec=need[2], weight_mode=RAD, r_cut=wl.r_cut)


def _check(eq, wl, gout, unsorted=False, perm_seed=2026, need=(True, True, True), what="", vec=None):
    vec = wl.vec if vec is None else vec
    ref = oracle.conv_backward_radial(wl.N, vec, wl.src, wl.dst, wl.x, wl.w_rad, gout, wl.lmax, wl.r_cut,
                                      wl.path_set)
    if unsorted:
        perm = np.random.default_rng(perm_seed).permutation(wl.src.shape[0])
        gx, gw, gv = _run(eq, wl, vec[perm], wl.src[perm], wl.dst[perm], gout, True, need)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.shape[0])
        gv_np = _np(gv)[inv] if gv is not None else None
    else:
        gx, gw, gv = _run(eq, wl, vec, wl.src, wl.dst, gout, False, need)
        gv_np = _np(gv) if gv is not None else None
    errs = []
    for got, r, name, want in ((gx, ref[0], "grad_x", need[0]), (gw, ref[1], "grad_W", need[1]),
                               (gv_np, ref[2], "grad_vec", need[2])):
        if not want:
            assert got is None
            continue
        got = got if isinstance(got, np.ndarray) else _np(got)
        assert got.shape == r.shape, (name, got.shape, r.shape)
        errs.append(_assert_close(got, r, TOL, what + " " + name))
    return errs


@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", [0, 1])
@pytest.mark.parametrize("C", [16, 32, 64, 128])
def test_radial_backward_small_sorted(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(37, 9, C, lmax, 900 + lmax * 10 + C + ps, path_set=ps, radial=True, r_cut=5.0,
                           empty_rows=(3,), long_rows=(5,), long_len=70, zero_vec_edges=1)
    _say("radial backward sorted lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.src.shape[0]))
    _check(eq, wl, _gout(wl, 7), what="sorted L%d ps%d C%d" % (lmax, ps, C))


@pytest.mark.parametrize("lmax,ps,C", [(3, 0, 128), (3, 1, 32), (2, 0, 16), (1, 1, 64), (0, 0, 16)])
def test_radial_backward_small_unsorted(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(41, 10, C, lmax, 950 + lmax + C, path_set=ps, radial=True, r_cut=5.0, empty_rows=(0,),
                           zero_vec_edges=2)
    _say("radial backward unsorted lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.src.shape[0]))
    _check(eq, wl, _gout(wl, 8), unsorted=True, what="unsorted L%d ps%d C%d" % (lmax, ps, C))


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True),
                                  (False, True, True)])
@pytest.mark.parametrize("unsorted", [False, True])
def test_radial_backward_partial_requests(need, unsorted):
    eq = _eq()
    wl = synth.small_graph(23, 8, 32, 3, 977, radial=True, r_cut=5.0)
    _say("radial backward partial %s unsorted=%s" % (need, unsorted))
    _check(eq, wl, _gout(wl, 9), unsorted=unsorted, need=need, what="partial")


def test_radial_backward_short_long_and_cut_edges():
    """Edge lengths across the radial basis' domain: near zero (the series branch of the
    derivative), around a r = 1/2 where the two branches meet, beyond r_c (no weight, no
    gradient), and exactly zero."""
    eq = _eq()
    wl = synth.small_graph(29, 12, 64, 3, 981, radial=True, r_cut=5.0)
    E = wl.src.shape[0]
    rng = np.random.default_rng(5)
    u = wl.vec / np.maximum(np.linalg.norm(wl.vec, axis=1, keepdims=True), 1e-30)
    lengths = np.linalg.norm(wl.vec, axis=1)
    kinds = rng.integers(0, 5, size=E)
    lengths = np.where(kinds == 0, rng.uniform(1e-4, 1e-2, E), lengths)
    lengths = np.where(kinds == 1, rng.uniform(0.05, 1.2, E), lengths)   # n pi r / r_c near 1/2 for some n
    lengths = np.where(kinds == 2, rng.uniform(5.0, 7.0, E), lengths)    # at or past the cutoff
    vec = (u * lengths[:, None]).astype(np.float32)
    vec[kinds == 3] = 0.0
    _say("radial backward lengths E=%d" % E)
    _check(eq, wl, _gout(wl, 11), vec=vec, what="lengths")
    _check(eq, wl, _gout(wl, 12), vec=vec, unsorted=True, what="lengths unsorted")


def test_radial_backward_no_edges():
    eq = _eq()
    import torch

    wl = synth.small_graph(6, 0, 16, 3, 983, radial=True, r_cut=5.0, empty_rows=range(6))
    assert wl.src.shape[0] == 0
    gout = _gout(wl, 13)
    gx, gw, gv = _run(eq, wl, wl.vec, wl.src, wl.dst, gout, False, (True, True, True))
    torch.cuda.synchronize()
    assert np.all(_np(gx) == 0.0) and np.all(_np(gw) == 0.0) and gv.shape == (0, 3)


def test_radial_backward_radial_workload_full():
    """The radial workload (50k atoms, r_c = 5 A, 2.6M edges, L = 3, C = 128): every entry of the three
    gradients, dst-sorted edges, against the oracle over all edges (its source blocks shared out over the
    host's threads)."""
    eq = _eq()
    wl = synth.make_config("radial")
    gout = _gout(wl, 14)
    _say("radial backward radial workload E=%d" % wl.src.shape[0])
    errs = _check(eq, wl, gout, what="radial workload")
    _say("radial workload rel errors %s" % (errs,))


@pytest.mark.parametrize("unsorted", [False, True])
def test_radial_autograd_function(unsorted):
    """equivariant_conv with radial weights: forward and the three gradients through torch.autograd."""
    import torch

    eq = _eq()
    from spherical_harmonic_cg_amd.autograd import equivariant_conv

    wl = synth.small_graph(19, 7, 32, 3, 990 + int(unsorted), radial=True, r_cut=5.0, zero_vec_edges=1)
    gout = _gout(wl, 15)
    vec = _t(wl.vec).requires_grad_(True)
    x = _t(wl.x).requires_grad_(True)
    W = _t(wl.w_rad).requires_grad_(True)
    kw = dict(dst=_t(wl.dst)) if unsorted else dict(row_ptr=_t(wl.row_ptr))
    _say("radial autograd unsorted=%s" % unsorted)
    out = equivariant_conv(vec, x, W, _t(wl.src), 3, weight_mode=RAD, r_cut=wl.r_cut, **kw)
    ref_out = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, 3, weight_mode=1, r_cut=wl.r_cut)
    _assert_close(_np(out.detach()), ref_out, TOL, "radial autograd forward")
    (out * _t(gout)).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.conv_backward_radial(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, gout, 3, wl.r_cut)
    _assert_close(_np(x.grad), ref[0], TOL, "radial autograd grad_x")
    _assert_close(_np(W.grad), ref[1], TOL, "radial autograd grad_W")
    _assert_close(_np(vec.grad), ref[2], TOL, "radial autograd grad_vec")
