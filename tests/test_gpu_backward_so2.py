"""GPU parity of the gradients in the edge-aligned (SO(2)) form
(eqtp_conv_backward with fixed weights at lmax 4..6, or EQTP_ALGO_EDGE_SO2 at
any lmax, through the C ABI) against the fp64 oracle's gradients, which come
from the Clebsch-Gordan definition and the harmonics' own gradient: the
kernel evaluates neither (it rotates the features into each edge's frame and
uses the generators of rotations for grad_vec).

Bar: max|gpu - oracle| <= 2e-4 * max|oracle| per gradient tensor (grad_x,
grad_w, grad_vec).  Cases: every lmax 0..6, both path sets, every supported
channel count, dst-sorted and unsorted edges, zero-length edges, edges along
+z / -z and nearly along z, empty and long rows, partial requests, and a
1,000-atom radius graph at lmax 6.
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _say, _t

pytestmark = pytest.mark.gpu

SO2 = 3


def _graph(L, ps, C, seed, n=23, deg=7):
    wl = synth.small_graph(n, deg, C, L, seed, path_set=ps, empty_rows=(2,), long_rows=(5,), long_len=70,
                           zero_vec_edges=2)
    wl.vec[2] = (0.0, 0.0, 1.7)
    wl.vec[3] = (0.0, 0.0, -0.9)
    wl.vec[4] = (1e-4, -2e-4, 1.3)
    wl.vec[5] = (3e-4, 1e-4, -2.2)
    return wl


def _gout(N, C, L, seed):
    return np.random.default_rng(seed).standard_normal((N, C, (L + 1) ** 2)).astype(np.float32)


def _run(eq, wl, w, gout, unsorted, algo=SO2, need=(True, True, True), perm_seed=5):
    kw = dict(path_set=wl.path_set, algo=algo, need_x=need[0], need_w=need[1], need_vec=need[2])
    if unsorted:
        perm = np.random.default_rng(perm_seed).permutation(wl.src.shape[0])
        gx, gw, gv = eq.eqtp_conv_backward(_t(wl.vec[perm]), _t(wl.src[perm]), _t(wl.x), _t(w), _t(gout), wl.lmax,
                                           dst=_t(wl.dst[perm]), **kw)
        if gv is not None:
            inv = np.empty_like(perm)
            inv[perm] = np.arange(perm.shape[0])
            gv = _np(gv)[inv]
        return gx, gw, gv
    return eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(w), _t(gout), wl.lmax,
                                 row_ptr=_t(wl.row_ptr), **kw)


def _compare(got, ref, need, what):
    for g, r, name, want in zip(got, ref, ("grad_x", "grad_w", "grad_vec"), need):
        if not want:
            assert g is None
            continue
        _assert_close(g if isinstance(g, np.ndarray) else _np(g), r, TOL, what + " " + name)


# C = 128 above lmax 4 runs as two launches over 64-channel halves
CASES = [(L, ps, C) for L in range(7) for ps in (0, 1) for C in (8, 16, 32, 64, 128)]


@pytest.mark.parametrize("L,ps,C", CASES)
def test_so2_backward_sorted(L, ps, C):
    eq = _eq()
    wl = _graph(L, ps, C, 2000 + 10 * L + C + ps)
    gout = _gout(wl.N, C, L, 31 + L)
    _say("so2 backward sorted L=%d ps=%d C=%d E=%d" % (L, ps, C, wl.src.shape[0]))
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, L, ps)
    _compare(_run(eq, wl, wl.w, gout, False), ref, (True, True, True), "so2 bwd L%d ps%d C%d" % (L, ps, C))


@pytest.mark.parametrize("L,ps,C", [(4, 0, 32), (5, 1, 16), (6, 0, 64), (6, 1, 8), (4, 1, 128), (5, 0, 128),
                                    (6, 1, 128), (3, 0, 64), (2, 1, 32), (0, 0, 16)])
def test_so2_backward_unsorted(L, ps, C):
    eq = _eq()
    wl = _graph(L, ps, C, 2100 + 10 * L + C + ps)
    gout = _gout(wl.N, C, L, 41 + L)
    _say("so2 backward unsorted L=%d ps=%d C=%d E=%d" % (L, ps, C, wl.src.shape[0]))
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, L, ps)
    _compare(_run(eq, wl, wl.w, gout, True), ref, (True, True, True), "so2 bwd unsorted L%d ps%d C%d" % (L, ps, C))


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True),
                                  (False, True, True)])
def test_so2_backward_partial_requests(need):
    eq = _eq()
    wl = _graph(5, 0, 32, 2201)
    gout = _gout(wl.N, 32, 5, 51)
    _say("so2 backward partial %s" % (need,))
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, 5, 0)
    _compare(_run(eq, wl, wl.w, gout, False, algo=0, need=need), ref, need, "so2 bwd partial")


@pytest.mark.parametrize("L", [4, 6])
def test_so2_backward_auto_for_high_lmax(L):
    """lmax above 3 with the default algorithm takes the edge-aligned gradients."""
    eq = _eq()
    wl = _graph(L, 1, 16, 2300 + L)
    gout = _gout(wl.N, 16, L, 61)
    _say("so2 backward auto L=%d" % L)
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, L, 1)
    _compare(_run(eq, wl, wl.w, gout, False, algo=0), ref, (True, True, True), "so2 bwd auto L%d" % L)


def test_so2_backward_rejects_unsupported():
    eq = _eq()
    _say("so2 backward unsupported combinations")
    wl = _graph(4, 0, 32, 8)
    gout = _gout(wl.N, 32, 4, 2)
    W = np.zeros((8, wl.w.size), dtype=np.float32)
    with pytest.raises(eq.EqtpError):                  # radial weights above lmax 3
        eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(W), _t(gout), 4, row_ptr=_t(wl.row_ptr),
                              weight_mode=eq.EQTP_W_RADIAL, r_cut=5.0)


def test_so2_backward_no_edges():
    eq = _eq()
    wl = synth.small_graph(6, 0, 32, 5, 2401, empty_rows=range(6))
    gout = _gout(wl.N, 32, 5, 3)
    _say("so2 backward no edges")
    gx, gw, gv = _run(eq, wl, wl.w, gout, False, algo=0)
    assert np.all(_np(gx) == 0.0) and np.all(_np(gw) == 0.0) and _np(gv).shape == (0, 3)


def test_so2_backward_lmax6_graph_full():
    """A 1,000-atom radius graph at lmax 6 (27 k edges, C = 32, parity paths): every entry of the
    three gradients against the oracle, dst-sorted and in random order."""
    eq = _eq()
    wl = synth.lmax_graph(6, 32, seed=11, n=1000)
    gout = _gout(wl.N, 32, 6, 71)
    _say("so2 backward lmax 6 graph E=%d" % wl.E)
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.weights, gout, 6, wl.path_set)
    g = eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.weights), _t(gout), 6,
                              row_ptr=_t(wl.row_ptr), path_set=wl.path_set)
    _compare(g, ref, (True, True, True), "so2 bwd L6 graph sorted")
    perm = np.random.default_rng(9).permutation(wl.E)
    gx, gw, gv = eq.eqtp_conv_backward(_t(wl.vec[perm]), _t(wl.src[perm]), _t(wl.x), _t(wl.weights), _t(gout), 6,
                                       dst=_t(wl.dst[perm]), path_set=wl.path_set)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(wl.E)
    _compare((gx, gw, _np(gv)[inv]), ref, (True, True, True), "so2 bwd L6 graph unsorted")


@pytest.mark.parametrize("L,csr", [(4, True), (6, False)])
def test_so2_autograd_high_lmax(L, csr):
    """equivariant_conv above lmax 3: the edge-aligned forward and gradients through torch.autograd
    (the default source-grouped mode falls back to eqtp_conv_backward there)."""
    eq = _eq()
    from spherical_harmonic_cg_amd.autograd import equivariant_conv

    wl = _graph(L, 0, 32, 2500 + L)
    gout = _gout(wl.N, 32, L, 81)
    kw = dict(row_ptr=_t(wl.row_ptr)) if csr else dict(dst=_t(wl.dst))
    vec = _t(wl.vec).requires_grad_(True)
    x = _t(wl.x).requires_grad_(True)
    w = _t(wl.w).requires_grad_(True)
    _say("so2 autograd L=%d csr=%s" % (L, csr))
    out = equivariant_conv(vec, x, w, _t(wl.src), L, **kw)
    _assert_close(_np(out.detach()), oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, L), TOL,
                  "so2 autograd forward")
    (out * _t(gout)).sum().backward()
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, L, 0)
    _compare((x.grad, w.grad, vec.grad), ref, (True, True, True), "so2 autograd L%d" % L)
