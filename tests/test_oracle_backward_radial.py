"""Pins for the oracle's gradients of the radial-weight convolution (CPU only).

oracle_conv_backward_radial is checked against facts that do not use its
formulas:
  * the envelope and radial-basis derivatives against central differences of
    oracle_envelope / oracle_radial_basis, and their zeros at r = 0 and r_c;
  * dL/dx and dL/dW by the adjoint identity: L is linear in x and in W, so
    <gx, dx> = <gout, conv(dx)> and <gW, dW> = <gout, conv(W = dW)> exactly;
  * dL/dvec by central differences of the forward oracle (radial mode) in
    fp64, edge by edge;
  * with every edge of one length r0 the radial weights are the fixed weights
    w = sum_b R_b(r0) W_b: grad_x and the tangential part of grad_vec equal the
    fixed-weight oracle's, and gW_b = R_b(r0) gw;
  * the result does not depend on the thread count (bit for bit).
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth

RC = 5.0


def _L(N, vec, src, dst, x, W, gout, lmax, ps, r_cut=RC):
    out = oracle.conv(N, vec, src, dst, x, W, lmax, path_set=ps, weight_mode=1, r_cut=r_cut)
    return float(np.sum(gout * out))


def _case(lmax, ps, seed, C=3, n=7, deg=4, zero_vec_edges=0):
    wl = synth.small_graph(n, deg, C, lmax, seed, path_set=ps, radial=True, r_cut=RC,
                           zero_vec_edges=zero_vec_edges)
    rng = np.random.default_rng(seed + 303)
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    gout = rng.standard_normal((wl.N, C, (lmax + 1) ** 2))
    return wl.N, f64(wl.vec), wl.src, wl.dst, f64(wl.x), f64(wl.w_rad), gout


def test_envelope_deriv_central_differences():
    h = 1e-6
    for d in np.linspace(0.02, 0.98, 25):
        fd = (oracle.envelope(d + h) - oracle.envelope(d - h)) / (2 * h)
        assert abs(oracle.envelope_deriv(d) - fd) < 1e-8
    assert oracle.envelope_deriv(0.0) == 0.0
    assert oracle.envelope_deriv(1.0) == 0.0 and oracle.envelope_deriv(1.7) == 0.0
    # u' vanishes at d = 1 from the left too (a zero of order 2 of u')
    assert abs(oracle.envelope_deriv(1.0 - 1e-9)) < 1e-14


@pytest.mark.parametrize("r_cut", [3.0, 5.0])
def test_radial_basis_deriv_central_differences(r_cut):
    h = 1e-6
    for r in np.linspace(0.05, 0.99 * r_cut, 30):
        fd = (oracle.radial_basis(r + h, r_cut, 8) - oracle.radial_basis(r - h, r_cut, 8)) / (2 * h)
        np.testing.assert_allclose(oracle.radial_basis_deriv(r, r_cut, 8), fd, rtol=0, atol=2e-7)
    assert np.all(oracle.radial_basis_deriv(0.0, r_cut, 8) == 0.0)
    assert np.all(oracle.radial_basis_deriv(r_cut * 1.2, r_cut, 8) == 0.0)
    assert np.abs(oracle.radial_basis_deriv(r_cut * (1 - 1e-9), r_cut, 8)).max() < 1e-12
    # near r = 0: sin(a r)/r = a - a^3 r^2 / 6 + ..., so the derivative is -a^3 r / 3 to first order
    a = np.arange(1, 9) * np.pi / r_cut
    np.testing.assert_allclose(oracle.radial_basis_deriv(1e-4, r_cut, 8), -a ** 3 * 1e-4 / 3, rtol=1e-5)


@pytest.mark.parametrize("lmax,ps", [(1, 0), (2, 0), (3, 0), (2, 1), (3, 1)])
def test_radial_backward_x_and_W_adjoint(lmax, ps):
    N, vec, src, dst, x, W, gout = _case(lmax, ps, 21 + lmax + 7 * ps)
    gx, gW, _ = oracle.conv_backward_radial(N, vec, src, dst, x, W, gout, lmax, RC, ps)
    rng = np.random.default_rng(7)
    for _ in range(3):
        dx = rng.standard_normal(x.shape)
        rhs = _L(N, vec, src, dst, dx, W, gout, lmax, ps)
        assert abs(float(np.sum(gx * dx)) - rhs) <= 1e-12 * max(1.0, abs(rhs))
        dW = rng.standard_normal(W.shape)
        rhs = _L(N, vec, src, dst, x, dW, gout, lmax, ps)
        assert abs(float(np.sum(gW * dW)) - rhs) <= 1e-12 * max(1.0, abs(rhs))


@pytest.mark.parametrize("lmax,ps", [(1, 0), (2, 0), (3, 0), (3, 1)])
def test_radial_backward_vec_central_differences(lmax, ps):
    N, vec, src, dst, x, W, gout = _case(lmax, ps, 41 + lmax)
    _, _, gv = oracle.conv_backward_radial(N, vec, src, dst, x, W, gout, lmax, RC, ps)
    rng = np.random.default_rng(9)
    h = 1e-5
    for _ in range(3):
        d = rng.standard_normal(vec.shape)
        fd = (_L(N, vec + h * d, src, dst, x, W, gout, lmax, ps) -
              _L(N, vec - h * d, src, dst, x, W, gout, lmax, ps)) / (2 * h)
        assert abs(float(np.sum(gv * d)) - fd) <= 1e-7 * max(1.0, abs(fd))
    for e in range(0, vec.shape[0], max(1, vec.shape[0] // 6)):
        for a in range(3):
            d = np.zeros_like(vec)
            d[e, a] = 1.0
            fd = (_L(N, vec + h * d, src, dst, x, W, gout, lmax, ps) -
                  _L(N, vec - h * d, src, dst, x, W, gout, lmax, ps)) / (2 * h)
            assert abs(gv[e, a] - fd) <= 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("lmax,ps", [(2, 0), (3, 0), (3, 1)])
def test_radial_backward_equal_lengths_is_fixed_weights(lmax, ps):
    N, vec, src, dst, x, W, gout = _case(lmax, ps, 61 + lmax, C=4, n=9)
    r0 = 2.3
    vec = vec / np.linalg.norm(vec, axis=1, keepdims=True) * r0
    R = oracle.radial_basis(r0, RC, 8)
    P = W.shape[1] // x.shape[1]
    w_fixed = (R @ W).reshape(P, x.shape[1])
    gx, gW, gv = oracle.conv_backward_radial(N, vec, src, dst, x, W, gout, lmax, RC, ps)
    fx, fw, fv = oracle.conv_backward(N, vec, src, dst, x, w_fixed, gout, lmax, ps)
    scale = max(1.0, np.abs(fx).max())
    np.testing.assert_allclose(gx, fx, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(gW, np.outer(R, fw.ravel()), rtol=0, atol=1e-12 * max(1.0, np.abs(fw).max()))
    u = vec / r0
    tangential = gv - np.sum(gv * u, axis=1, keepdims=True) * u
    np.testing.assert_allclose(tangential, fv, rtol=0, atol=1e-11 * max(1.0, np.abs(fv).max()))


def test_radial_backward_zero_length_edges():
    N, vec, src, dst, x, W, gout = _case(3, 0, 71, zero_vec_edges=2)
    assert np.all(vec[:2] == 0.0)
    gx, gW, gv = oracle.conv_backward_radial(N, vec, src, dst, x, W, gout, 3, RC, 0)
    assert np.all(gv[:2] == 0.0)
    rng = np.random.default_rng(3)
    dx = rng.standard_normal(x.shape)
    assert abs(np.sum(gx * dx) - _L(N, vec, src, dst, dx, W, gout, 3, 0)) < 1e-11
    dW = rng.standard_normal(W.shape)
    assert abs(np.sum(gW * dW) - _L(N, vec, src, dst, x, dW, gout, 3, 0)) < 1e-11


def test_radial_backward_edges_beyond_cutoff_have_no_radial_term():
    # beyond r_c every R_b and R_b' is 0: the convolution and every gradient vanish
    N, vec, src, dst, x, W, gout = _case(2, 0, 81)
    vec = vec / np.linalg.norm(vec, axis=1, keepdims=True) * (RC * 1.5)
    gx, gW, gv = oracle.conv_backward_radial(N, vec, src, dst, x, W, gout, 2, RC, 0)
    assert np.all(gx == 0.0) and np.all(gW == 0.0) and np.all(gv == 0.0)


def test_radial_backward_thread_count_independent():
    wl = synth.small_graph(2600, 3, 2, 2, 91, radial=True, r_cut=RC)  # three blocks of source nodes
    gout = np.random.default_rng(4).standard_normal((wl.N, 2, 9)).astype(np.float32)
    try:
        oracle.set_threads(1)
        a = oracle.conv_backward_radial(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, gout, 2, RC)
        oracle.set_threads(5)
        b = oracle.conv_backward_radial(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, gout, 2, RC)
    finally:
        oracle.set_threads(0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_radial_backward_float32_entry_and_subsets():
    wl = synth.small_graph(6, 5, 4, 3, 95, radial=True, r_cut=RC)
    gout = np.random.default_rng(2).standard_normal((wl.N, 4, 16)).astype(np.float32)
    a = oracle.conv_backward_radial(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, gout, 3, RC)
    b = oracle.conv_backward_radial(wl.N, wl.vec.astype(np.float64), wl.src, wl.dst, wl.x.astype(np.float64),
                                    wl.w_rad.astype(np.float64), gout.astype(np.float64), 3, RC)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    for need in [(True, False, False), (False, True, False), (False, False, True)]:
        c = oracle.conv_backward_radial(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, gout, 3, RC, need=need)
        for i in range(3):
            assert (c[i] is None) != need[i]
            if need[i]:
                assert np.array_equal(c[i], a[i])


def test_radial_backward_rejects_out_of_range_index():
    wl = synth.small_graph(5, 3, 2, 1, 97, radial=True, r_cut=RC)
    src = wl.src.copy()
    src[0] = wl.N
    gout = np.zeros((wl.N, 2, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.conv_backward_radial(wl.N, wl.vec, src, wl.dst, wl.x, wl.w_rad, gout, 1, RC)


def test_radial_basis_deriv_series_branch_is_continuous():
    # a r = 1e-2 switches between the Taylor series and the closed form; dR/r is smooth there
    # (-a^3/3 (1 - (a r)^2 / 10 + ...) times u ~ 1), so both sides of the switch agree on it
    r_cut = 5.0
    for n in (1, 4, 8):
        a = n * np.pi / r_cut
        r_lo, r_hi = 0.9999999e-2 / a, 1.0000001e-2 / a
        lo = oracle.radial_basis_deriv(r_lo, r_cut, 8)[n - 1] / r_lo
        hi = oracle.radial_basis_deriv(r_hi, r_cut, 8)[n - 1] / r_hi
        assert abs(lo - hi) <= 1e-10 * abs(lo)
        assert abs(lo - (-a ** 3 / 3) * (1 - 1e-4 / 10)) <= 1e-8 * abs(lo)
