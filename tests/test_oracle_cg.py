"""Pins for the oracle's Clebsch-Gordan coefficients and path sets (CPU only).

Independent routes: sympy's exact Clebsch-Gordan routine (a textbook table),
unitarity, the Gaunt integral of three real spherical harmonics computed by
quadrature, and the along-z special case that relates the real-basis block to
the complex coefficients with m2 = 0.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _triples(lmax):
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
                yield l1, l2, l3


def _sympy_cg(l1, m1, l2, m2, l3, m3):
    from sympy import N as numeric
    from sympy.physics.wigner import clebsch_gordan

    return float(numeric(clebsch_gordan(l1, l2, l3, m1, m2, m3), 30))


def test_complex_cg_vs_sympy():
    """Racah formula == sympy's exact clebsch_gordan for every l <= 3 entry
    (and a few l = 5, 6 ones)."""
    checked = 0
    for l1, l2, l3 in _triples(3):
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                m3 = m1 + m2
                if abs(m3) > l3:
                    continue
                a = oracle.cg_complex(l1, m1, l2, m2, l3, m3)
                b = _sympy_cg(l1, m1, l2, m2, l3, m3)
                assert abs(a - b) < 1e-13, (l1, m1, l2, m2, l3, m3, a, b)
                checked += 1
    for args in [(5, 2, 6, -1, 4, 1), (6, 3, 6, -3, 0, 0), (5, -5, 5, 5, 7, 0), (6, 0, 3, 2, 7, 2)]:
        assert abs(oracle.cg_complex(*args) - _sympy_cg(*args)) < 1e-13
    assert checked == 478  # every (l1,l2,l3 <= 3, m1, m2) entry


def test_complex_cg_selection_rules():
    assert oracle.cg_complex(1, 1, 1, 0, 2, 0) == 0.0  # m3 != m1 + m2
    assert oracle.cg_complex(1, 0, 1, 0, 3, 0) == 0.0  # triangle violated


@pytest.mark.parametrize("l1,l2", [(1, 1), (2, 1), (2, 3), (3, 3)])
def test_complex_cg_unitarity(l1, l2):
    """The CG matrix from |l1 m1> |l2 m2> to |l3 m3> is orthogonal."""
    rows = []
    for l3 in range(abs(l1 - l2), l1 + l2 + 1):
        for m3 in range(-l3, l3 + 1):
            rows.append([oracle.cg_complex(l1, m1, l2, m2, l3, m3)
                         for m1 in range(-l1, l1 + 1) for m2 in range(-l2, l2 + 1)])
    M = np.array(rows)
    n = (2 * l1 + 1) * (2 * l2 + 1)
    assert M.shape == (n, n)
    np.testing.assert_allclose(M @ M.T, np.eye(n), atol=1e-13)


@pytest.mark.parametrize("l1,l2", [(0, 3), (1, 2), (2, 2), (3, 3), (3, 2), (4, 3), (5, 4), (6, 6), (6, 1)])
def test_real_cg_unitarity_and_discard(l1, l2):
    """Real-basis blocks for all l3 stack into an orthogonal matrix, and the
    dropped part (imag for even, real for odd l1+l2+l3) vanishes."""
    rows = []
    for l3 in range(abs(l1 - l2), l1 + l2 + 1):
        c, disc = oracle.cg_real(l1, l2, l3, return_discard=True)
        assert disc < 1e-14
        for mu3 in range(2 * l3 + 1):
            rows.append(c[:, :, mu3].reshape(-1))
    M = np.array(rows)
    np.testing.assert_allclose(M @ M.T, np.eye(M.shape[0]), atol=1e-13)


def test_identity_paths():
    """C(0,l,l) and C(l,0,l) are identities; C(1,1,0) = -I/sqrt3."""
    for l in range(4):
        np.testing.assert_allclose(oracle.cg_real(0, l, l)[0], np.eye(2 * l + 1), atol=1e-15)
        np.testing.assert_allclose(oracle.cg_real(l, 0, l)[:, 0, :], np.eye(2 * l + 1), atol=1e-15)
    np.testing.assert_allclose(oracle.cg_real(1, 1, 0)[:, :, 0], -np.eye(3) / math.sqrt(3), atol=1e-15)


def _quadrature_grid(nz=8, nphi=12):
    zg, wg = np.polynomial.legendre.leggauss(nz)
    phi = 2 * np.pi * np.arange(nphi) / nphi
    Z, PH = np.meshgrid(zg, phi, indexing="ij")
    s = np.sqrt(1 - Z ** 2)
    dirs = np.stack([s * np.cos(PH), s * np.sin(PH), Z], axis=-1).reshape(-1, 3)
    wts = (wg[:, None] * np.full(nphi, 2 * np.pi / nphi)[None, :]).reshape(-1)
    return dirs, wts


def _closed_form_sh(v):
    """Real SH l <= 3 from textbook polynomials (own copy, unit vectors, fp64)."""
    from test_oracle_sh import _closed_forms

    return _closed_forms(v)


def test_real_cg_gaunt_relation():
    """For even l1+l2+l3:  integral of Y_mu1 Y_mu2 Y_mu3 over the sphere
    = sqrt((2l1+1)(2l2+1) / (4 pi (2l3+1))) <l1 0 l2 0|l3 0> C[mu1,mu2,mu3],
    with <l1 0 l2 0|l3 0> from sympy and the integral by exact quadrature on
    fp64 closed-form harmonics (no complex-to-real change of basis involved)."""
    dirs, wts = _quadrature_grid()
    Y = _closed_form_sh(dirs)
    checked = 0
    for l1, l2, l3 in _triples(3):
        if (l1 + l2 + l3) % 2:
            continue
        Y1 = Y[:, l1 * l1:(l1 + 1) ** 2]
        Y2 = Y[:, l2 * l2:(l2 + 1) ** 2]
        Y3 = Y[:, l3 * l3:(l3 + 1) ** 2]
        gaunt = np.einsum("q,qa,qb,qc->abc", wts, Y1, Y2, Y3)
        k = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (4 * math.pi * (2 * l3 + 1))) * _sympy_cg(l1, 0, l2, 0, l3, 0)
        np.testing.assert_allclose(gaunt, k * oracle.cg_real(l1, l2, l3), atol=1e-14, err_msg=str((l1, l2, l3)))
        checked += 1
    assert checked == 23


def test_real_cg_along_z():
    """With m2 = 0 only (an edge along +z), the real block reduces to the complex
    coefficient <l1 m l2 0 | l3 m>:
      even l1+l2+l3: C[c_m,0,c_m] = C[s_m,0,s_m] = <l1 m l2 0|l3 m>, C[0,0,0] = <l1 0 l2 0|l3 0>;
      odd  l1+l2+l3: C[c_m,0,s_m] = -<l1 m l2 0|l3 m>, C[s_m,0,c_m] = +<l1 m l2 0|l3 m>.
    Checked against sympy; this fixes each path's sign."""
    for l1, l2, l3 in _triples(3):
        C = oracle.cg_real(l1, l2, l3)
        odd = (l1 + l2 + l3) % 2
        for m in range(0, min(l1, l3) + 1):
            ref = _sympy_cg(l1, m, l2, 0, l3, m)
            if m == 0:
                assert abs(C[0, 0, 0] - (0.0 if odd else ref)) < 1e-14
                continue
            c1, s1, c3, s3 = 2 * m - 1, 2 * m, 2 * m - 1, 2 * m
            if not odd:
                assert abs(C[c1, 0, c3] - ref) < 1e-14
                assert abs(C[s1, 0, s3] - ref) < 1e-14
                assert abs(C[c1, 0, s3]) < 1e-14 and abs(C[s1, 0, c3]) < 1e-14
            else:
                assert abs(C[c1, 0, s3] + ref) < 1e-14
                assert abs(C[s1, 0, c3] - ref) < 1e-14
                assert abs(C[c1, 0, c3]) < 1e-14 and abs(C[s1, 0, s3]) < 1e-14


@pytest.mark.parametrize("lmax", [5, 6])
def test_real_cg_along_z_high_l(lmax):
    """The along-z reduction for every path with max(l1, l2, l3) = lmax (the
    blocks the edge-aligned form uses at high degree), against sympy."""
    for l1, l2, l3 in _triples(lmax):
        if max(l1, l2, l3) != lmax:
            continue
        C = oracle.cg_real(l1, l2, l3)
        odd = (l1 + l2 + l3) % 2
        for m in range(0, min(l1, l3) + 1):
            ref = _sympy_cg(l1, m, l2, 0, l3, m)
            if m == 0:
                assert abs(C[0, 0, 0] - (0.0 if odd else ref)) < 1e-13
                continue
            c1, s1 = 2 * m - 1, 2 * m
            if not odd:
                assert abs(C[c1, 0, c1] - ref) < 1e-13 and abs(C[s1, 0, s1] - ref) < 1e-13
            else:
                assert abs(C[c1, 0, s1] + ref) < 1e-13 and abs(C[s1, 0, c1] - ref) < 1e-13
        # nothing couples different |m| through the m = 0 harmonic
        for a in range(2 * l1 + 1):
            for c in range(2 * l3 + 1):
                if (a + 1) // 2 != (c + 1) // 2:
                    assert abs(C[a, 0, c]) < 1e-14


def test_levi_civita_path():
    """(1,1,1) couples like the cross product: in Cartesian order (x, y, z) the
    real block is proportional to the Levi-Civita symbol with |entries| 1/sqrt2."""
    C = oracle.cg_real(1, 1, 1)
    # page order within l=1 is (z, -x, -y) up to the positive factor sqrt(3/4pi)
    P = np.array([[0, 0, 1], [-1, 0, 0], [0, -1, 0]], dtype=float)  # page <- cartesian
    Cc = np.einsum("ai,bj,ck,abc->ijk", P, P, P, C)
    eps = np.zeros((3, 3, 3))
    for i, j, k, s in [(0, 1, 2, 1), (1, 2, 0, 1), (2, 0, 1, 1), (0, 2, 1, -1), (2, 1, 0, -1), (1, 0, 2, -1)]:
        eps[i, j, k] = s
    scale = Cc[0, 1, 2]
    assert abs(abs(scale) - 1 / math.sqrt(2)) < 1e-14
    np.testing.assert_allclose(Cc, scale * eps, atol=1e-14)


def test_real_cg_entries_are_sqrt_rationals():
    """Every non-zero entry squared is a rational with a small denominator."""
    from fractions import Fraction

    mags = set()
    for l1, l2, l3 in _triples(3):
        for v in oracle.cg_real(l1, l2, l3).ravel():
            if abs(v) < 1e-14:
                continue
            f = Fraction(v * v).limit_denominator(10000)
            assert abs(float(f) - v * v) < 1e-13
            assert f.denominator <= 10000
            mags.add(f)
    assert len(mags) > 10


def _read_kv(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                d[k] = int(v)
    return d


def test_page_path_count():
    """The page's constexpr array for L_MAX = 3 has 34 entries: the SO(3) path set."""
    g = _read_kv("page_path_count.txt")
    assert len(oracle.paths(g["lmax"], oracle.PATHS_SO3)) == g["paths_so3"]


def test_path_sets():
    p = oracle.paths(3, oracle.PATHS_PARITY)
    assert len(p) == 23
    assert all((a + b + c) % 2 == 0 for a, b, c in p)
    assert [tuple(r) for r in p[:6]] == [(0, 0, 0), (0, 1, 1), (0, 2, 2), (0, 3, 3), (1, 0, 1), (1, 1, 0)]
    # lexicographic order
    assert [tuple(r) for r in p] == sorted(tuple(r) for r in p)
    assert len(oracle.paths(2, oracle.PATHS_PARITY)) == 11
    assert len(oracle.paths(2, oracle.PATHS_SO3)) == 15


def test_nnz_counts():
    def nnz(L, s):
        return sum(int((np.abs(oracle.cg_real(*p)) > 1e-12).sum()) for p in oracle.paths(L, s))

    assert nnz(3, 0) == 353
    assert nnz(3, 1) == 611
    assert nnz(2, 0) == 83
    assert nnz(2, 1) == 137
