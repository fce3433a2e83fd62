"""Pins for the oracle's interaction layer (CPU only): channel linear, radial
MLP, convolution with per-edge weights from the MLP, channel linear.

  * SiLU at closed-form points;
  * the radial network vanishes beyond the cutoff (R = 0, SiLU(0) = 0), depends
    on the edge length only, and with one hidden unit and unit weights is
    SiLU(SiLU(R_1(r)));
  * the convolution with a per-edge basis equals the radial-weight convolution
    when the basis is the radial functions themselves (same arithmetic, bit for
    bit) and the fixed-weight convolution when the basis is the same on every
    edge;
  * the layer with identity linears and norm 1 is that convolution, and the
    output scales as 1 / norm;
  * the whole layer is rotation-equivariant: rotating every edge vector by Q and
    every feature block of degree l by D_l(Q) rotates the output by D_l(Q),
    with D_l(Q) fitted from the harmonics themselves (Y_l(Q u) = D_l(Q) Y_l(u));
    a wrong coupling coefficient, path, sign or index breaks this.
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth

RC = 5.0


def test_silu_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), abs=1e-16)
    assert oracle.silu(-1.0) == pytest.approx(-1.0 / (1.0 + np.e), abs=1e-16)
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15


def _graph(lmax, ps, seed, C=3, n=9, deg=4):
    wl = synth.small_graph(n, deg, C, lmax, seed, path_set=ps, radial=True, r_cut=RC)
    iw = synth.interaction_weights(lmax, C, ps, H=6, seed=seed)
    return wl, iw


def test_radial_mlp_beyond_cutoff_is_zero_and_length_only():
    wl, iw = _graph(2, 0, 11)
    vec = wl.vec.astype(np.float64)
    far = vec / np.linalg.norm(vec, axis=1, keepdims=True) * (RC * 1.3)
    assert np.all(oracle.radial_mlp(far, RC, iw.W1, iw.W2) == 0.0)
    # a rotation of the edge vectors leaves the network's output unchanged
    q, _ = np.linalg.qr(np.random.default_rng(3).standard_normal((3, 3)))
    a = oracle.radial_mlp(vec, RC, iw.W1, iw.W2)
    b = oracle.radial_mlp(vec @ q.T, RC, iw.W1, iw.W2)
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-13)


def test_radial_mlp_single_unit():
    vec = np.array([[0.3, 1.1, -0.2], [2.0, 0.0, 0.0], [0.0, 0.0, 0.0]])
    W1 = np.zeros((8, 1))
    W1[0, 0] = 1.0
    phi = oracle.radial_mlp(vec, RC, W1, np.ones((1, 1)))
    for e in range(3):
        r = float(np.linalg.norm(vec[e]))
        want = oracle.silu(oracle.silu(oracle.radial_basis(r, RC, 8)[0]))
        assert phi[e, 0] == pytest.approx(want, rel=1e-15, abs=1e-300)


@pytest.mark.parametrize("lmax,ps", [(1, 0), (2, 1), (3, 0), (3, 1)])
def test_conv_basis_is_radial_conv_when_basis_is_radial(lmax, ps):
    wl, _ = _graph(lmax, ps, 21 + lmax)
    vec = wl.vec.astype(np.float64)
    r = np.sqrt(vec[:, 0] * vec[:, 0] + vec[:, 1] * vec[:, 1] + vec[:, 2] * vec[:, 2])
    phi = np.stack([oracle.radial_basis(float(ri), RC, 8) for ri in r]) if len(r) else np.zeros((0, 8))
    x = wl.x.astype(np.float64)
    W = wl.w_rad.astype(np.float64)
    a = oracle.conv_basis(wl.N, vec, wl.src, wl.dst, x, phi, W, lmax, ps)
    b = oracle.conv(wl.N, vec, wl.src, wl.dst, x, W, lmax, path_set=ps, weight_mode=1, r_cut=RC)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("lmax,ps", [(2, 0), (3, 1)])
def test_conv_basis_constant_basis_is_fixed_weights(lmax, ps):
    wl, iw = _graph(lmax, ps, 31 + lmax)
    E, C = wl.src.shape[0], wl.C
    P = synth.num_paths(lmax, ps)
    phi0 = np.random.default_rng(5).standard_normal(6)
    phi = np.tile(phi0, (E, 1))
    W3 = iw.W3.astype(np.float64)
    a = oracle.conv_basis(wl.N, wl.vec, wl.src, wl.dst, wl.x.astype(np.float64), phi, W3, lmax, ps)
    w_fixed = (phi0 @ W3).reshape(P, C)
    b = oracle.conv(wl.N, wl.vec.astype(np.float64), wl.src, wl.dst, wl.x.astype(np.float64), w_fixed, lmax,
                    path_set=ps)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13 * max(1.0, np.abs(b).max()))


@pytest.mark.parametrize("lmax,ps", [(1, 0), (3, 0)])
def test_interaction_identity_linears_and_norm(lmax, ps):
    wl, iw = _graph(lmax, ps, 41 + lmax)
    C = wl.C
    eye = np.broadcast_to(np.eye(C), (lmax + 1, C, C)).astype(np.float64).copy()
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    vec = f64(wl.vec)
    out = oracle.interaction(wl.N, vec, wl.src, wl.dst, f64(wl.x), eye, f64(iw.W1), f64(iw.W2), f64(iw.W3), eye,
                             lmax, RC)
    phi = oracle.radial_mlp(vec, RC, iw.W1, iw.W2)
    ref = oracle.conv_basis(wl.N, vec, wl.src, wl.dst, f64(wl.x), phi, f64(iw.W3), lmax, ps)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13 * max(1.0, np.abs(ref).max()))
    half = oracle.interaction(wl.N, vec, wl.src, wl.dst, f64(wl.x), eye, f64(iw.W1), f64(iw.W2), f64(iw.W3), eye,
                              lmax, RC, norm=2.0)
    np.testing.assert_allclose(half, out / 2.0, rtol=0, atol=1e-15 * max(1.0, np.abs(out).max()))


def _wigner_from_harmonics(q, lmax, rng):
    """D_l(Q) for l = 0..lmax, the matrices with Y_l(Q u) = D_l(Q) Y_l(u), by least squares over random
    directions."""
    u = rng.standard_normal((60, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    Y = oracle.sh(u, lmax)
    Yq = oracle.sh(u @ q.T, lmax)
    D = []
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        sol, *_ = np.linalg.lstsq(Y[:, sl], Yq[:, sl], rcond=None)  # Y D^T = Yq
        D.append(sol.T)
    return D


def _rotate_features(x, D):
    out = np.empty_like(x)
    for l, Dl in enumerate(D):
        sl = slice(l * l, (l + 1) * (l + 1))
        out[:, :, sl] = x[:, :, sl] @ Dl.T
    return out


@pytest.mark.parametrize("lmax,ps", [(1, 0), (2, 0), (3, 0), (3, 1)])
def test_interaction_rotation_equivariant(lmax, ps):
    wl, iw = _graph(lmax, ps, 51 + lmax + 5 * ps, C=4, n=11, deg=5)
    rng = np.random.default_rng(77 + lmax)
    q, _ = np.linalg.qr(rng.standard_normal((3, 3)))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]  # a proper rotation
    D = _wigner_from_harmonics(q, lmax, rng)
    for Dl in D:  # the fit is an orthogonal matrix
        np.testing.assert_allclose(Dl @ Dl.T, np.eye(Dl.shape[0]), atol=1e-12)
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    args = (f64(iw.W_up), f64(iw.W1), f64(iw.W2), f64(iw.W3), f64(iw.W_out), lmax, RC)
    vec, x = f64(wl.vec), f64(wl.x)
    out = oracle.interaction(wl.N, vec, wl.src, wl.dst, x, *args, norm=3.0, path_set=ps)
    out_rot = oracle.interaction(wl.N, vec @ q.T, wl.src, wl.dst, _rotate_features(x, D), *args, norm=3.0,
                                 path_set=ps)
    np.testing.assert_allclose(out_rot, _rotate_features(out, D), rtol=0,
                               atol=1e-11 * max(1.0, np.abs(out).max()))


def test_interaction_float32_entry_matches_widened():
    wl, iw = _graph(3, 0, 61, C=4)
    a = oracle.interaction(wl.N, wl.vec, wl.src, wl.dst, wl.x, iw.W_up, iw.W1, iw.W2, iw.W3, iw.W_out, 3, RC,
                           norm=2.5)
    f64 = lambda t: np.asarray(t, dtype=np.float64)
    b = oracle.interaction(wl.N, f64(wl.vec), wl.src, wl.dst, f64(wl.x), f64(iw.W_up), f64(iw.W1), f64(iw.W2),
                           f64(iw.W3), f64(iw.W_out), 3, RC, norm=2.5)
    assert np.array_equal(a, b)
