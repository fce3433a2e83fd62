"""Pins for the oracle's real spherical harmonics (CPU only).

Each test checks the oracle against something other than itself: the values
printed on the Batmobile page, a closed-form identity, scipy's complex
spherical harmonics, or a quadrature.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit_dirs(n, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((n, 3))
    return (v / np.linalg.norm(v, axis=1, keepdims=True)).astype(np.float32)


def _read_page_constants():
    rows = []
    with open(os.path.join(GOLDEN, "page_sh_constants.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, coef, var = line.split()
            rows.append((name, float(coef), var))
    return rows


# index of each named component in the page's declaration order
PAGE_INDEX = {"Y00": 0, "Y10": 1, "Y11c": 2, "Y11s": 3}


def test_page_constants_by_name():
    """Y00, Y10, Y11c, Y11s equal the page's printed formulas."""
    v = _unit_dirs(200, 1)
    Y = oracle.sh(v, 1)
    vd = v.astype(np.float64)
    vd /= np.linalg.norm(vd, axis=1, keepdims=True)
    var = {"1": np.ones(len(v)), "nx": vd[:, 0], "ny": vd[:, 1], "nz": vd[:, 2]}
    for name, coef, vname in _read_page_constants():
        np.testing.assert_allclose(Y[:, PAGE_INDEX[name]], coef * var[vname], rtol=0, atol=1e-15, err_msg=name)


def test_page_constants_unnormalised_input():
    """The page normalises the edge vector before evaluating: the result does
    not depend on the vector's length."""
    v = _unit_dirs(50, 2)
    for lmax in (1, 3, 5):
        a = oracle.sh(v, lmax)
        b = oracle.sh(v * np.float32(4.0), lmax)  # exact scaling in float32
        np.testing.assert_allclose(a, b, atol=1e-14)


@pytest.mark.parametrize("lmax", [0, 1, 2, 3, 6])
def test_addition_theorem(lmax):
    """sum_m Y_lm^2 = (2l+1)/(4 pi) for every direction."""
    Y = oracle.sh(_unit_dirs(300, 3), lmax)
    for l in range(lmax + 1):
        s = (Y[:, l * l:(l + 1) ** 2] ** 2).sum(axis=1)
        np.testing.assert_allclose(s, (2 * l + 1) / (4 * math.pi), rtol=1e-13)


def test_addition_theorem_values():
    """The four per-l constants at L=3 (0.0795775, 0.2387324, 0.3978874, 0.5570423)."""
    Y = oracle.sh(_unit_dirs(10, 4), 3)
    want = [0.0795775, 0.2387324, 0.3978874, 0.5570423]
    for l in range(4):
        s = (Y[:, l * l:(l + 1) ** 2] ** 2).sum(axis=1)
        np.testing.assert_allclose(s, want[l], atol=5e-8)


@pytest.mark.parametrize("lmax", [3, 6])
def test_against_scipy_complex_sh(lmax):
    """Real SH = (Re, Im) of scipy's complex SH (Condon-Shortley phase) times sqrt2
    for m > 0, in the page's (l0, l1c, l1s, l2c, l2s, ...) order."""
    from scipy.special import sph_harm_y

    v = _unit_dirs(100, 5).astype(np.float64)
    theta = np.arccos(np.clip(v[:, 2], -1, 1))
    phi = np.arctan2(v[:, 1], v[:, 0])
    Y = oracle.sh(v.astype(np.float32), lmax)
    # recompute angles from the float32 vectors the oracle saw
    vf = v.astype(np.float32).astype(np.float64)
    vf /= np.linalg.norm(vf, axis=1, keepdims=True)
    theta = np.arccos(np.clip(vf[:, 2], -1, 1))
    phi = np.arctan2(vf[:, 1], vf[:, 0])
    for l in range(lmax + 1):
        np.testing.assert_allclose(Y[:, l * l], sph_harm_y(l, 0, theta, phi).real, atol=1e-13)
        for m in range(1, l + 1):
            z = sph_harm_y(l, m, theta, phi)
            np.testing.assert_allclose(Y[:, l * l + 2 * m - 1], math.sqrt(2) * z.real, atol=1e-13)
            np.testing.assert_allclose(Y[:, l * l + 2 * m], math.sqrt(2) * z.imag, atol=1e-13)


def _closed_forms(v):
    """Textbook polynomial forms of the real SH for l <= 3 (unit vector)."""
    x, y, z = v[:, 0], v[:, 1], v[:, 2]
    pi = math.pi
    out = np.empty((len(v), 16))
    out[:, 0] = 0.5 / math.sqrt(pi)
    c1 = math.sqrt(3 / (4 * pi))
    out[:, 1], out[:, 2], out[:, 3] = c1 * z, -c1 * x, -c1 * y
    out[:, 4] = math.sqrt(5 / (16 * pi)) * (3 * z * z - 1)
    c21 = math.sqrt(15 / (4 * pi))
    out[:, 5], out[:, 6] = -c21 * x * z, -c21 * y * z
    c22 = math.sqrt(15 / (16 * pi))
    out[:, 7], out[:, 8] = c22 * (x * x - y * y), 2 * c22 * x * y
    out[:, 9] = math.sqrt(7 / (16 * pi)) * z * (5 * z * z - 3)
    c31 = math.sqrt(21 / (32 * pi))
    out[:, 10], out[:, 11] = -c31 * x * (5 * z * z - 1), -c31 * y * (5 * z * z - 1)
    c32 = math.sqrt(105 / (16 * pi))
    out[:, 12], out[:, 13] = c32 * z * (x * x - y * y), 2 * c32 * x * y * z
    c33 = math.sqrt(35 / (32 * pi))
    out[:, 14], out[:, 15] = -c33 * x * (x * x - 3 * y * y), -c33 * y * (3 * x * x - y * y)
    return out


def test_closed_forms_l3():
    v = _unit_dirs(300, 6)
    vd = v.astype(np.float64)
    vd /= np.linalg.norm(vd, axis=1, keepdims=True)
    np.testing.assert_allclose(oracle.sh(v, 3), _closed_forms(vd), atol=2e-15)


def test_closed_form_constants_printed():
    """Spot values of the l=2,3 constants (derived, not printed on the page)."""
    assert abs(math.sqrt(5 / (16 * math.pi)) - 0.31539156525252005) < 1e-16
    assert abs(math.sqrt(15 / (4 * math.pi)) - 1.0925484305920792) < 1e-15
    assert abs(math.sqrt(7 / (16 * math.pi)) - 0.3731763325901154) < 1e-16
    assert abs(math.sqrt(35 / (32 * math.pi)) - 0.5900435899266435) < 1e-16
    assert abs(math.sqrt(3 / (4 * math.pi)) - 0.4886025119029199) < 1e-16


def test_orthonormal_by_quadrature():
    """Gauss-Legendre in cos(theta) x uniform phi integrates products of
    degree <= 12 exactly: <Y_a, Y_b> = delta_ab for all l <= 6."""
    lmax = 6
    zg, wg = np.polynomial.legendre.leggauss(16)
    nphi = 32
    phi = 2 * np.pi * np.arange(nphi) / nphi
    Z, PH = np.meshgrid(zg, phi, indexing="ij")
    s = np.sqrt(1 - Z ** 2)
    dirs = np.stack([s * np.cos(PH), s * np.sin(PH), Z], axis=-1).reshape(-1, 3)
    wts = (wg[:, None] * np.full(nphi, 2 * np.pi / nphi)[None, :]).reshape(-1)
    # float32 directions lose precision; evaluate on the float32-rounded points
    Y = oracle.sh(dirs.astype(np.float32), lmax)
    G = (Y * wts[:, None]).T @ Y
    np.testing.assert_allclose(G, np.eye(G.shape[0]), atol=2e-6)


def test_zero_vector():
    """A zero-length edge keeps only Y00 (reading of a case the page leaves open)."""
    Y = oracle.sh(np.zeros((3, 3), np.float32), 3)
    assert np.all(Y[:, 0] == 0.5 / math.sqrt(math.pi))
    assert np.all(Y[:, 1:] == 0.0)


def test_inversion_parity():
    """Y_l(-r) = (-1)^l Y_l(r)."""
    v = _unit_dirs(100, 7)
    a, b = oracle.sh(v, 5), oracle.sh(-v, 5)
    for l in range(6):
        np.testing.assert_allclose(b[:, l * l:(l + 1) ** 2], (-1) ** l * a[:, l * l:(l + 1) ** 2], atol=1e-14)


def test_axis_values():
    """Along +z only the m=0 components survive, equal to sqrt((2l+1)/(4pi))."""
    Y = oracle.sh(np.array([[0, 0, 2.5]], np.float32), 6)[0]
    for l in range(7):
        assert abs(Y[l * l] - math.sqrt((2 * l + 1) / (4 * math.pi))) < 1e-14
        assert np.all(np.abs(Y[l * l + 1:(l + 1) ** 2]) < 1e-14)
