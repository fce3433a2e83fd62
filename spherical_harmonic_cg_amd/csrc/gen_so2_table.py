#!/usr/bin/env python3
"""Build step: tables for the edge-aligned (SO(2)) form of the convolution.

Writes ``generated/so2_tables.inc`` next to this file (checked in, like the
Clebsch-Gordan tables of gen_cg_table.py, whose exact arithmetic it reuses).

What the edge-aligned form needs (E2Former-V2 page, section 2.1 "derivation
of EAAS"): rotate the node features into a frame whose z axis is the edge
direction; there the harmonics of the edge keep only their m = 0 component,
so the coupling becomes a sparse re-indexing in which each output component
receives at most a couple of input components of the same |m|.

* Coupling: for every path (l1, l2, l3) the real-basis coefficients with the
  harmonic component (l2, m = 0), multiplied by Y_{l2,0}(z axis) =
  sqrt((2 l2 + 1) / (4 pi)), exact in Decimal then rounded to float32.
* Frame rotation: D(R) with Y(R u) = D(R) Y(u) for the real harmonics in the
  page's component order.  R = R_y(-theta) R_z(-phi) takes the edge direction
  (theta, phi) to the z axis; D(R_z(a)) is a 2x2 rotation by m a of each
  (m cos, m sin) pair, and D(R_y(b)) = J^T D(R_z(b)) J with the constant
  J = D(R_x(pi/2)).  J is obtained from its defining property by a least
  squares fit on sample directions (float64; its entries are algebraic
  numbers, and the fit is checked to be orthogonal and exact to 1e-12),
  then rounded to float32.
* Every table is checked here: the rotation property of the harmonics, the
  equivariance of the Clebsch-Gordan tables under D, and that the sparse
  coupling after rotation equals the full coupling for random inputs.
* Harmonic prefactors for degrees up to 6 (standalone evaluation by the
  Legendre-derivative recurrence): sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!), times
  sqrt2 (-1)^m for m > 0.
* Rotation generators for the gradient with respect to the edge vector:
  L_a = d/de D(R_a(e)) at e = 0 for a = x, y (antisymmetric, block diagonal,
  sparse), from L_z (each (m cos, m sin) pair: (-m v_s, m v_c)) as
  L_y = J^T L_z J and L_x = D_y L_z D_y^T with D_y = D(R_y(pi/2)) =
  J^T D(R_z(pi/2)) J.  Checked against central differences of fitted D, and
  the identity the gradient kernel uses is checked against finite
  differences of the harmonics (see check_gradient).
"""
from __future__ import annotations

import hashlib
import math
import os
import sys
from decimal import Decimal

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import gen_cg_table as cg  # noqa: E402  (exact Racah / real-basis arithmetic)

OUT = os.path.join(HERE, "generated", "so2_tables.inc")
LMAX_SO2 = 6


def real_sh(u, lmax):
    """Real harmonics [n, (lmax+1)^2] of unit vectors [n, 3] in the page's
    order (per l: m = 0, then (m cos, m sin) for m = 1..l), Condon-Shortley
    phase kept: Y_lm,c = sqrt2 N_lm P_l^m(z) cos(m phi), Y_lm,s = ... sin."""
    x, y, z = u[:, 0], u[:, 1], u[:, 2]
    phi = np.arctan2(y, x)
    s = np.sqrt(np.maximum(0.0, 1.0 - z * z))
    out = np.zeros((u.shape[0], (lmax + 1) ** 2))
    # associated Legendre with the (-1)^m phase, by the standard recurrences
    P = {}
    P[(0, 0)] = np.ones_like(z)
    for m in range(1, lmax + 1):
        P[(m, m)] = -(2 * m - 1) * s * P[(m - 1, m - 1)]
    for m in range(0, lmax):
        P[(m + 1, m)] = (2 * m + 1) * z * P[(m, m)]
    for m in range(0, lmax + 1):
        for l in range(m + 2, lmax + 1):
            P[(l, m)] = ((2 * l - 1) * z * P[(l - 1, m)] - (l + m - 1) * P[(l - 2, m)]) / (l - m)
    for l in range(lmax + 1):
        for m in range(l + 1):
            N = math.sqrt((2 * l + 1) / (4 * math.pi) * math.factorial(l - m) / math.factorial(l + m))
            if m == 0:
                out[:, l * l] = N * P[(l, 0)]
            else:
                out[:, l * l + 2 * m - 1] = math.sqrt(2) * N * P[(l, m)] * np.cos(m * phi)
                out[:, l * l + 2 * m] = math.sqrt(2) * N * P[(l, m)] * np.sin(m * phi)
    return out


def rot_x(a):
    c, s = math.cos(a), math.sin(a)
    return np.array([[1, 0, 0], [0, c, -s], [0, s, c]])


def rot_y(a):
    c, s = math.cos(a), math.sin(a)
    return np.array([[c, 0, s], [0, 1, 0], [-s, 0, c]])


def rot_z(a):
    c, s = math.cos(a), math.sin(a)
    return np.array([[c, -s, 0], [s, c, 0], [0, 0, 1]])


def sample_dirs(n, seed):
    v = np.random.default_rng(seed).standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def wigner_fit(Rm, lmax):
    """Block-diagonal D with Y(R u) = D Y(u), fitted on sample directions."""
    u = sample_dirs(400, 1)
    A = real_sh(u, lmax)            # [n, K]
    B = real_sh(u @ Rm.T, lmax)     # Y(R u)
    D = np.linalg.lstsq(A, B, rcond=None)[0].T
    K = (lmax + 1) ** 2
    blk = np.zeros((K, K))
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        blk[sl, sl] = D[sl, sl]
    assert np.abs(D - blk).max() < 1e-10, "rotation mixes different l"
    assert np.abs(blk @ blk.T - np.eye(K)).max() < 1e-12, "fitted D is not orthogonal"
    assert np.abs(A @ blk.T - B).max() < 1e-12, "fit residual"
    return blk


def z_rot(a, lmax):
    """D(R_z(a)): 2x2 rotation of each (m cos, m sin) pair by m a."""
    K = (lmax + 1) ** 2
    D = np.zeros((K, K))
    for l in range(lmax + 1):
        D[l * l, l * l] = 1.0
        for m in range(1, l + 1):
            c, s = l * l + 2 * m - 1, l * l + 2 * m
            D[c, c] = math.cos(m * a)
            D[c, s] = -math.sin(m * a)
            D[s, c] = math.sin(m * a)
            D[s, s] = math.cos(m * a)
    return D


def gen_z(lmax):
    """L_z = d/da D(R_z(a)) at a = 0."""
    K = (lmax + 1) ** 2
    G = np.zeros((K, K))
    for l in range(lmax + 1):
        for m in range(1, l + 1):
            c, s = l * l + 2 * m - 1, l * l + 2 * m
            G[c, s] = -m
            G[s, c] = m
    return G


def generators(J, lmax):
    """(L_x, L_y) in the real-harmonic basis, from J and L_z."""
    Lz = gen_z(lmax)
    Ly = J.T @ Lz @ J
    Dy = J.T @ z_rot(math.pi / 2, lmax) @ J
    Lx = Dy @ Lz @ Dy.T
    return Lx, Ly


def full_cg(lmax, path_set):
    """[(l1, l2, l3, dense real block as float64)] from the exact tables."""
    out = []
    for (l1, l2, l3) in cg.paths(lmax, path_set):
        blk = cg.real_block(l1, l2, l3)
        M = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
        for (a, b, c), (coef, sq) in blk.items():
            M[a, b, c] = float(cg.exact_decimal(coef, sq))
        out.append((l1, l2, l3, blk, M))
    return out


def so2_terms(cgl):
    """Sparse coupling with the harmonic fixed at the z axis: per path p the
    entries C[mu1, (l2, m=0), mu3] * Y_{l2,0}(z) as (p, mu1, mu3, l2, float32, text)."""
    pi = cg._pi()
    terms = []
    for p, (l1, l2, l3, blk, _) in enumerate(cgl):
        yz = (Decimal(2 * l2 + 1) / (4 * pi)).sqrt()
        for (a, b, c), (coef, sq) in sorted(blk.items()):
            if b != 0:
                continue
            val = cg.exact_decimal(coef, sq) * yz
            terms.append((p, l1 * l1 + a, l3 * l3 + c, l2, cg.nearest_f32(val),
                          "%s * sqrt(%d/(4 pi))" % (cg.surd_text(coef, sq), 2 * l2 + 1)))
    return terms


def check(lmax, path_set, J, cgl, terms):
    K = (lmax + 1) ** 2
    rng = np.random.default_rng(7)
    # the factorisation of D(R_y(b)) through J, and the z rotation, against fits
    for b in (0.3, -1.1, 2.5):
        assert np.abs(J.T @ z_rot(b, lmax) @ J - wigner_fit(rot_y(b), lmax)).max() < 1e-12
        assert np.abs(z_rot(b, lmax) - wigner_fit(rot_z(b), lmax)).max() < 1e-12
    # equivariance of the exact tables under a random rotation
    Rm = rot_z(0.7) @ rot_y(-1.3) @ rot_z(2.1)
    D = wigner_fit(Rm, lmax)
    for (l1, l2, l3, _, M) in cgl:
        D1 = D[l1 * l1:(l1 + 1) ** 2, l1 * l1:(l1 + 1) ** 2]
        D2 = D[l2 * l2:(l2 + 1) ** 2, l2 * l2:(l2 + 1) ** 2]
        D3 = D[l3 * l3:(l3 + 1) ** 2, l3 * l3:(l3 + 1) ** 2]
        a = rng.standard_normal(2 * l1 + 1)
        b = rng.standard_normal(2 * l2 + 1)
        lhs = np.einsum("ijk,i,j->k", M, D1 @ a, D2 @ b)
        rhs = D3 @ np.einsum("ijk,i,j->k", M, a, b)
        assert np.abs(lhs - rhs).max() < 1e-12, ("CG not equivariant", l1, l2, l3)
    # the edge-aligned product equals the full product with Y(u)
    for trial in range(5):
        u = sample_dirs(1, 100 + trial)[0]
        if trial == 0:
            u = np.array([0.0, 0.0, -1.0])
        theta = math.acos(max(-1.0, min(1.0, u[2])))
        phi = math.atan2(u[1], u[0])
        Dr = J.T @ z_rot(-theta, lmax) @ J @ z_rot(-phi, lmax)
        Y = real_sh(u[None, :], lmax)[0]
        assert np.abs(Dr @ Y - real_sh(np.array([[0.0, 0.0, 1.0]]), lmax)[0]).max() < 1e-12
        x = rng.standard_normal(K)
        w = rng.standard_normal(len(cgl))
        full = np.zeros(K)
        for p, (l1, l2, l3, _, M) in enumerate(cgl):
            full[l3 * l3:(l3 + 1) ** 2] += w[p] * np.einsum("ijk,i,j->k", M, x[l1 * l1:(l1 + 1) ** 2],
                                                            Y[l2 * l2:(l2 + 1) ** 2])
        xt = Dr @ x
        mt = np.zeros(K)
        for (p, mu1, mu3, l2, c, _) in terms:
            mt[mu3] += w[p] * c * xt[mu1]
        assert np.abs(Dr.T @ mt - full).max() < 1e-5 * max(1.0, np.abs(full).max()), "edge-aligned product"


def check_generators(J, lmax):
    K = (lmax + 1) ** 2
    Lx, Ly = generators(J, lmax)
    eps = 1e-4
    for G, rot in ((Lx, rot_x), (Ly, rot_y)):
        fd = (wigner_fit(rot(eps), lmax) - wigner_fit(rot(-eps), lmax)) / (2 * eps)
        assert np.abs(G - fd).max() < 1e-6, "generator against central differences"
        assert np.abs(G + G.T).max() < 1e-12, "generator not antisymmetric"
    # L_z itself, and the pole derivatives: d/dx Y(z axis) = L_y Y(z axis), d/dy Y(z axis) = -L_x Y(z axis)
    fd = (wigner_fit(rot_z(eps), lmax) - wigner_fit(rot_z(-eps), lmax)) / (2 * eps)
    assert np.abs(gen_z(lmax) - fd).max() < 1e-6
    y0 = real_sh(np.array([[0.0, 0.0, 1.0]]), lmax)[0]
    h = 1e-4  # the harmonics' own evaluation limits the difference quotient near the pole to ~1e-7
    for a, want in ((0, Ly @ y0), (1, -(Lx @ y0))):
        e = np.zeros(3)
        e[a] = h
        up, dn = np.array([[0.0, 0.0, 1.0]]) + e, np.array([[0.0, 0.0, 1.0]]) - e
        d = (real_sh(up / np.linalg.norm(up), lmax)[0] - real_sh(dn / np.linalg.norm(dn), lmax)[0]) / (2 * h)
        assert np.abs(d - want).max() < 1e-6 * max(1.0, np.abs(want).max()), "pole derivative"
    return Lx, Ly


def check_gradient(lmax, J, Lx, Ly, cgl, terms):
    """The gradient of L = g . out_e with respect to the edge vector, computed
    in the edge frame as the kernel does, against central differences of the
    full coupling: with x' = D x, g' = D g (D = D(R_e)), u' = P_w x' (the
    message in the frame) and v' = P_w^T g',
        G_x = -(v' . L_y x' + u' . L_y g'),  G_y = v' . L_x x' + u' . L_x g',
        dL/dvec = R_e^T (G_x, G_y, 0) / |vec|."""
    K = (lmax + 1) ** 2
    rng = np.random.default_rng(11)

    def loss(vec, x, g, w):
        u = vec / np.linalg.norm(vec)
        Y = real_sh(u[None, :], lmax)[0]
        out = np.zeros(K)
        for p, (l1, l2, l3, _, M) in enumerate(cgl):
            out[l3 * l3:(l3 + 1) ** 2] += w[p] * np.einsum("ijk,i,j->k", M, x[l1 * l1:(l1 + 1) ** 2],
                                                           Y[l2 * l2:(l2 + 1) ** 2])
        return g @ out

    for trial in range(4):
        vec = rng.standard_normal(3) * 2.0
        x, g, w = rng.standard_normal(K), rng.standard_normal(K), rng.standard_normal(len(cgl))
        r = np.linalg.norm(vec)
        theta = math.acos(vec[2] / r)
        phi = math.atan2(vec[1], vec[0])
        Dr = J.T @ z_rot(-theta, lmax) @ J @ z_rot(-phi, lmax)
        xt, gt = Dr @ x, Dr @ g
        P = np.zeros((K, K))  # P_w[mu3, mu1]
        for (p, mu1, mu3, l2, c, _) in terms:
            P[mu3, mu1] += w[p] * c
        ut, vt = P @ xt, P.T @ gt
        gx = -(vt @ (Ly @ xt) + ut @ (Ly @ gt))
        gy = vt @ (Lx @ xt) + ut @ (Lx @ gt)
        Re = rot_y(-theta) @ rot_z(-phi)
        grad = Re.T @ np.array([gx, gy, 0.0]) / r
        h = 1e-6
        fd = np.array([(loss(vec + h * np.eye(3)[a], x, g, w) - loss(vec - h * np.eye(3)[a], x, g, w)) / (2 * h)
                       for a in range(3)])
        assert np.abs(grad - fd).max() < 1e-6 * max(1.0, np.abs(fd).max()), ("edge-frame gradient", lmax, grad, fd)


def sparse_rows(M):
    ent = []
    for r in range(M.shape[0]):
        for c in range(M.shape[1]):
            if abs(M[r, c]) > 1e-12:
                ent.append((r, c, float(np.float32(M[r, c]))))
    starts = [next((i for i, e in enumerate(ent) if e[0] >= r), len(ent)) for r in range(M.shape[0] + 1)]
    return ent, starts


def main(out_path: str = OUT):
    src_hash = hashlib.sha256(open(os.path.abspath(__file__), "rb").read()).hexdigest()[:16]
    lines = []
    w = lines.append
    w("// Generated by gen_so2_table.py (source sha256 %s). Do not edit." % src_hash)
    w("// Edge-aligned (SO(2)) form of the convolution, components in the page's")
    w("// order (per l: l0, l1c, l1s, l2c, l2s, ...).")
    w("#pragma once")
    w("")
    w("namespace eqtp_gen {")
    w("")
    w("struct So2Term {")
    w("  unsigned char p, mu1, mu3, l2;  // path, feature component, output component, harmonic l")
    w("  float c;                        // C^p[mu1, (l2, m=0), mu3] * Y_{l2,0}(z axis)")
    w("};")
    w("")
    w("struct JEntry {")
    w("  unsigned char row, col;  // indices into the (lmax+1)^2 vector")
    w("  float v;")
    w("};")
    w("")
    Jfull = wigner_fit(rot_x(math.pi / 2), LMAX_SO2)
    Jent = []
    for r in range(Jfull.shape[0]):
        for c in range(Jfull.shape[1]):
            v = Jfull[r, c]
            if abs(v) > 1e-12:
                Jent.append((r, c, float(np.float32(v))))
    w("// J = D(R_x(pi/2)) for l <= %d (block diagonal), non-zero entries by row" % LMAX_SO2)
    w("constexpr int kJNumEntries = %d;" % len(Jent))
    w("constexpr JEntry kJ[%d] = {" % len(Jent))
    for (r, c, v) in Jent:
        w("    {%d, %d, %s}," % (r, c, cg.f32_literal(v)))
    w("};")
    nrow = Jfull.shape[0]
    starts = [next((i for i, e in enumerate(Jent) if e[0] >= r), len(Jent)) for r in range(nrow + 1)]
    w("// first entry of each row, and one past the last row")
    w("constexpr short kJRowStart[%d] = {%s};" % (nrow + 1, ", ".join(str(s) for s in starts)))
    JTent = sorted(((c, r, v) for (r, c, v) in Jent))
    w("// J^T (= J^-1), non-zero entries by row")
    w("constexpr JEntry kJT[%d] = {" % len(JTent))
    for (r, c, v) in JTent:
        w("    {%d, %d, %s}," % (r, c, cg.f32_literal(v)))
    w("};")
    startsT = [next((i for i, e in enumerate(JTent) if e[0] >= r), len(JTent)) for r in range(nrow + 1)]
    w("constexpr short kJTRowStart[%d] = {%s};" % (nrow + 1, ", ".join(str(s) for s in startsT)))
    w("")
    Lx, Ly = check_generators(Jfull, LMAX_SO2)
    for name, G, axis in (("kLx", Lx, "x"), ("kLy", Ly, "y")):
        ent, st = sparse_rows(G)
        w("// L_%s = d/de D(R_%s(e)) at e = 0 for l <= %d (antisymmetric), non-zero entries by row" % (
            axis, axis, LMAX_SO2))
        w("constexpr JEntry %s[%d] = {" % (name, len(ent)))
        for (r, c, v) in ent:
            w("    {%d, %d, %s}," % (r, c, cg.f32_literal(v)))
        w("};")
        w("constexpr short %sRowStart[%d] = {%s};" % (name, nrow + 1, ", ".join(str(x) for x in st)))
    w("")
    # harmonics of degree up to LMAX_SO2 for the standalone evaluation:
    #   Y_l0 = N_l0 Q_l^0(z),  Y_lm,c/s = sqrt2 (-1)^m N_lm Q_l^m(z) Re/Im (x + i y)^m
    # with Q_l^m = d^m P_l / dz^m and N_lm = sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!)
    pi = cg._pi()
    w("// real-harmonic prefactors A[l][m] (see sh.hip), nearest float32 of the exact value")
    w("constexpr float kShPrefactor[%d][%d] = {" % (LMAX_SO2 + 1, LMAX_SO2 + 1))
    for l in range(LMAX_SO2 + 1):
        vals = []
        for m in range(LMAX_SO2 + 1):
            if m > l:
                vals.append("0.0f")
                continue
            n2 = Decimal(2 * l + 1) / (4 * pi) * Decimal(math.factorial(l - m)) / Decimal(math.factorial(l + m))
            a = n2.sqrt() if m == 0 else (2 * n2).sqrt() * (-1 if m % 2 else 1)
            vals.append(cg.f32_literal(cg.nearest_f32(a)))
        w("    {%s}," % ", ".join(vals))
    w("};")
    w("")
    summary = []
    for path_set, psname in cg.PATH_SETS.items():
        for lmax in range(LMAX_SO2 + 1):
            cgl = full_cg(lmax, path_set)
            terms = so2_terms(cgl)
            K = (lmax + 1) ** 2
            check(lmax, path_set, Jfull[:K, :K], cgl, terms)
            check_gradient(lmax, Jfull[:K, :K], Lx[:K, :K], Ly[:K, :K], cgl, terms)
            tag = "L%d_%s" % (lmax, psname)
            nnz_full = sum(len(c[3]) for c in cgl)
            summary.append((tag, len(cgl), len(terms), nnz_full))
            w("// lmax = %d, %s path set: %d paths, %d edge-aligned terms (full coupling: %d)" % (
                lmax, psname, len(cgl), len(terms), nnz_full))
            w("constexpr int kSo2NumPaths_%s = %d;" % (tag, len(cgl)))
            w("constexpr int kSo2NumTerms_%s = %d;" % (tag, len(terms)))
            w("constexpr PathLs kSo2Paths_%s[%d] = {" % (tag, len(cgl)))
            for (l1, l2, l3, _, _) in cgl:
                w("    {%d, %d, %d}," % (l1, l2, l3))
            w("};")
            # by path, then output component: one weight per path, one run per (path, output)
            w("constexpr So2Term kSo2Terms_%s[%d] = {" % (tag, len(terms)))
            for t in sorted(terms, key=lambda t: (t[0], t[2], t[1])):
                w("    {%d, %d, %d, %d, %s},  // %s" % (t[0], t[1], t[2], t[3], cg.f32_literal(t[4]), t[5]))
            w("};")
            w("")
    w("}  // namespace eqtp_gen")
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    for tag, P, T, F in summary:
        print("%-12s paths %3d edge-aligned terms %4d (full coupling %5d)" % (tag, P, T, F))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1] if len(sys.argv) > 1 else OUT))
