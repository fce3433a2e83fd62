#!/usr/bin/env python3
"""Build step: exact real-basis Clebsch-Gordan tables for the HIP kernels.

Writes ``generated/cg_tables.inc`` next to this file.  Run it after changing
it; the output is checked in so that building the library needs no Python.

What it computes (Batmobile page, section "1. compile-time constants": the
coupling coefficients are mathematical constants baked into the kernel at
compile time, indexed by path):

* complex coefficients <l1 m1 l2 m2 | l3 m3> by the Racah formula in exact
  rational arithmetic: the value is S * sqrt(A) with S, A rational;
* the real basis of the page (section "2. register intermediate
  computation": per l the components are ordered l0, l1c, l1s, l2c, l2s, ...
  with Y_lm,c = sqrt2 Re Y_l^m, Y_lm,s = sqrt2 Im Y_l^m, Condon-Shortley phase
  kept), reached with the unitary change of basis U_l:
      C[mu1,mu2,mu3] = sum U_l3[mu3,m3] <l1m1 l2m2|l3m3> conj(U_l1[mu1,m1]) conj(U_l2[mu2,m2]);
  every term is (unit complex) * 2^(-k/2) * S * sqrt(A), so the sum is kept
  exactly as a combination of square roots of square-free integers;
* even l1+l2+l3 entries are real, odd ones purely imaginary (their imaginary
  part is used); every non-zero entry reduces to a single a*sqrt(b);
* paths (l1 = feature l, l2 = harmonic l, l3 = output l), triangle rule, all
  l <= lmax; the "parity" set keeps l1+l2+l3 even, the "so3" set keeps all;
  canonical order is lexicographic in (l1, l2, l3);
* float literals are the float32 values nearest to the exact entries.

Emitted per (lmax, path set): the path list, and the non-zero terms twice:
sorted by output component (for the node-side contraction) and by path
(for the per-edge product).
"""
from __future__ import annotations

import hashlib
import math
import os
import struct
import sys
from decimal import Decimal, getcontext
from fractions import Fraction

getcontext().prec = 60

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "generated", "cg_tables.inc")

LMAX_MAX = 3
PATH_SETS = {0: "parity", 1: "so3"}


def fact(n: int) -> int:
    return math.factorial(n)


def racah(l1, m1, l2, m2, l3, m3):
    """<l1 m1 l2 m2|l3 m3> = S * sqrt(A), returned as (S, A) Fractions."""
    if m3 != m1 + m2 or not (abs(l1 - l2) <= l3 <= l1 + l2):
        return Fraction(0), Fraction(0)
    if abs(m1) > l1 or abs(m2) > l2 or abs(m3) > l3:
        return Fraction(0), Fraction(0)
    A = Fraction((2 * l3 + 1) * fact(l1 + l2 - l3) * fact(l1 - l2 + l3) * fact(-l1 + l2 + l3),
                 fact(l1 + l2 + l3 + 1))
    A *= fact(l1 + m1) * fact(l1 - m1) * fact(l2 + m2) * fact(l2 - m2) * fact(l3 + m3) * fact(l3 - m3)
    S = Fraction(0)
    for k in range(0, l1 + l2 + l3 + 1):
        args = (l1 + l2 - l3 - k, l1 - m1 - k, l2 + m2 - k, l3 - l2 + m1 + k, l3 - l1 - m2 + k)
        if min(args) < 0:
            continue
        den = fact(k)
        for a in args:
            den *= fact(a)
        S += Fraction((-1) ** k, den)
    return S, A


def squarefree_split(q: Fraction):
    """sqrt(q) = c * sqrt(b) with c rational, b square-free integer."""
    if q == 0:
        return Fraction(0), 1
    n = q.numerator * q.denominator  # sqrt(n/d) = sqrt(n*d)/d
    c = Fraction(1, q.denominator)
    b = 1
    p = 2
    rest = n
    while p * p <= rest:
        while rest % (p * p) == 0:
            rest //= p * p
            c *= p
        if rest % p == 0:
            rest //= p
            b *= p
        p += 1
    b *= rest
    return c, b


class Surd:
    """Exact element of Q(i)(sqrt2, sqrt b...) kept as {b: complex-rational coef}:
    value = sum_b (re_b + i im_b) sqrt(b)."""

    def __init__(self):
        self.terms = {}

    def add(self, re: Fraction, im: Fraction, b: int):
        r0, i0 = self.terms.get(b, (Fraction(0), Fraction(0)))
        self.terms[b] = (r0 + re, i0 + im)

    def part(self, imag: bool):
        out = {}
        for b, (re, im) in self.terms.items():
            v = im if imag else re
            if v != 0:
                out[b] = v
        return out


def u_entry(l, mu, m):
    """U_l[mu][m] as (re, im, sqrt2_power) with value (re + i im) * 2^(-k/2)."""
    if mu == 0:
        return (Fraction(1), Fraction(0), 0) if m == 0 else None
    mm = (mu + 1) // 2
    is_sin = mu % 2 == 0
    sgn = -1 if mm % 2 else 1
    if m == mm:
        return (Fraction(0), Fraction(-1), 1) if is_sin else (Fraction(1), Fraction(0), 1)
    if m == -mm:
        return (Fraction(0), Fraction(sgn), 1) if is_sin else (Fraction(sgn), Fraction(0), 1)
    return None


def real_block(l1, l2, l3):
    """{(mu1,mu2,mu3): (coef Fraction, b)} non-zero exact entries; value coef*sqrt(b)."""
    odd = (l1 + l2 + l3) % 2 == 1
    out = {}
    for mu1 in range(2 * l1 + 1):
        for mu2 in range(2 * l2 + 1):
            for mu3 in range(2 * l3 + 1):
                s = Surd()
                for m1 in range(-l1, l1 + 1):
                    u1 = u_entry(l1, mu1, m1)
                    if u1 is None:
                        continue
                    for m2 in range(-l2, l2 + 1):
                        u2 = u_entry(l2, mu2, m2)
                        if u2 is None:
                            continue
                        m3 = m1 + m2
                        u3 = u_entry(l3, mu3, m3) if abs(m3) <= l3 else None
                        if u3 is None:
                            continue
                        S, A = racah(l1, m1, l2, m2, l3, m3)
                        if S == 0:
                            continue
                        # u3 * conj(u1) * conj(u2)
                        re, im = u3[0], u3[1]
                        for (ar, ai) in ((u1[0], -u1[1]), (u2[0], -u2[1])):
                            re, im = re * ar - im * ai, re * ai + im * ar
                        k = u1[2] + u2[2] + u3[2]
                        # 2^(-k/2) sqrt(A) S = S * sqrt(A / 2^k)
                        c, b = squarefree_split(A / Fraction(2 ** k))
                        s.add(re * S * c, im * S * c, b)
                vals = s.part(imag=odd)
                if not vals:
                    continue
                if len(vals) != 1:
                    raise RuntimeError("entry is not a single surd: %r" % vals)
                (b, coef), = vals.items()
                out[(mu1, mu2, mu3)] = (coef, b)
    # the discarded part must vanish identically
    return out


def exact_decimal(coef: Fraction, b: int) -> Decimal:
    return Decimal(coef.numerator) / Decimal(coef.denominator) * Decimal(b).sqrt()


def nearest_f32(x: Decimal) -> float:
    """float32 nearest to the exact value x (ties to even)."""
    f = struct.unpack("f", struct.pack("f", float(x)))[0]
    best = None
    bits = struct.unpack("I", struct.pack("f", f))[0]
    for db in (-1, 0, 1):
        cand = struct.unpack("f", struct.pack("I", (bits + db) & 0xffffffff))[0]
        err = abs(Decimal(cand) - x)
        key = (err, struct.unpack("I", struct.pack("f", cand))[0] & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def f32_literal(v: float) -> str:
    if v == 0.0:
        return "0.0f"
    return "%.9ef" % v


def paths(lmax, path_set):
    out = []
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(lmax + 1):
                if abs(l1 - l2) <= l3 <= l1 + l2 and (path_set == 1 or (l1 + l2 + l3) % 2 == 0):
                    out.append((l1, l2, l3))
    return out


def surd_text(coef: Fraction, b: int) -> str:
    q = coef * coef * b
    sign = "-" if coef < 0 else "+"
    return "%ssqrt(%s)" % (sign, q)


def build_terms(lmax, path_set):
    terms = []  # (p, mu1, mu2, mu3 global indices, float, text)
    for p, (l1, l2, l3) in enumerate(paths(lmax, path_set)):
        blk = real_block(l1, l2, l3)
        for (a, b, c), (coef, sq) in sorted(blk.items()):
            val = nearest_f32(exact_decimal(coef, sq))
            terms.append((p, l1 * l1 + a, l2 * l2 + b, l3 * l3 + c, val, surd_text(coef, sq)))
    return terms


# Decimal pi to 50 digits (Machin-type series), used for the SH norms.
def _pi() -> Decimal:
    getcontext().prec = 70

    def arctan_inv(n):
        x = Decimal(1) / n
        x2 = x * x
        total, term, k = Decimal(0), x, 1
        while term != 0:
            total += term / k if (k // 2) % 2 == 0 else -term / k
            term *= x2
            k += 2
        return total

    pi = 16 * arctan_inv(5) - 4 * arctan_inv(239)
    getcontext().prec = 60
    return +pi


# normalisation constants sqrt(a / (b pi)) of the real harmonics for l <= 3:
# Y_lm,c/s = sqrt2 N_lm P_l^m(cos t) cos/sin(m phi) written as polynomials in
# the unit vector (x, y, z); name -> (a, b)
SH_NORMS = [
    ("kShY00", 1, 4),     # Y00
    ("kShC1", 3, 4),      # Y10 = C1 z, Y11c = -C1 x, Y11s = -C1 y
    ("kShC20", 5, 16),    # Y20 = C20 (3 z^2 - 1)
    ("kShC21", 15, 4),    # Y21c = -C21 x z, Y21s = -C21 y z
    ("kShC22", 15, 16),   # Y22c = C22 (x^2 - y^2), Y22s = 2 C22 x y
    ("kShC30", 7, 16),    # Y30 = C30 z (5 z^2 - 3)
    ("kShC31", 21, 32),   # Y31c = -C31 x (5 z^2 - 1), Y31s = -C31 y (5 z^2 - 1)
    ("kShC32", 105, 16),  # Y32c = C32 z (x^2 - y^2), Y32s = 2 C32 x y z
    ("kShC33", 35, 32),   # Y33c = -C33 x (x^2 - 3 y^2), Y33s = -C33 y (3 x^2 - y^2)
]


def main(out_path: str = OUT):
    src_hash = hashlib.sha256(open(os.path.abspath(__file__), "rb").read()).hexdigest()[:16]
    lines = []
    w = lines.append
    w("// Generated by gen_cg_table.py (source sha256 %s). Do not edit." % src_hash)
    w("// Real-basis Clebsch-Gordan coefficients in the page's component order")
    w("// (per l: l0, l1c, l1s, l2c, l2s, ...), exact value in each comment.")
    w("// Term fields: p = path index, mu1 = feature component, mu2 = harmonic")
    w("// component, mu3 = output component (indices into the (lmax+1)^2 vector).")
    w("#pragma once")
    w("")
    w("namespace eqtp_gen {")
    w("")
    w("struct CgTerm {")
    w("  unsigned char p, mu1, mu2, mu3;")
    w("  float c;")
    w("};")
    w("")
    w("struct PathLs {")
    w("  unsigned char l1, l2, l3;")
    w("};")
    w("")
    pi = _pi()
    w("// real spherical harmonic normalisations sqrt(a / (b pi)), nearest float32")
    for name, a, b in SH_NORMS:
        val = (Decimal(a) / (Decimal(b) * pi)).sqrt()
        w("constexpr float %s = %s;  // sqrt(%d/(%d pi)) = %s" % (name, f32_literal(nearest_f32(val)), a, b,
                                                            str(val)[:22]))
    w("constexpr float kPiF = %s;" % f32_literal(nearest_f32(pi)))
    w("")
    summary = []
    for path_set, psname in PATH_SETS.items():
        for lmax in range(LMAX_MAX + 1):
            pl = paths(lmax, path_set)
            terms = build_terms(lmax, path_set)
            tag = "L%d_%s" % (lmax, psname)
            summary.append((tag, len(pl), len(terms)))
            w("// lmax = %d, %s path set: %d paths, %d non-zero coefficients" % (lmax, psname, len(pl), len(terms)))
            w("constexpr int kNumPaths_%s = %d;" % (tag, len(pl)))
            w("constexpr int kNumTerms_%s = %d;" % (tag, len(terms)))
            w("constexpr PathLs kPaths_%s[%d] = {" % (tag, len(pl)))
            for (l1, l2, l3) in pl:
                w("    {%d, %d, %d}," % (l1, l2, l3))
            w("};")
            for order_name, key in (("ByOut", lambda t: (t[3], t[0], t[1], t[2])),
                                    ("ByPath", lambda t: (t[0], t[3], t[1], t[2]))):
                w("constexpr CgTerm kTerms%s_%s[%d] = {" % (order_name, tag, len(terms)))
                for t in sorted(terms, key=key):
                    w("    {%d, %d, %d, %d, %s},  // %s" % (t[0], t[1], t[2], t[3], f32_literal(t[4]), t[5]))
                w("};")
            w("")
    w("}  // namespace eqtp_gen")
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    for tag, P, T in summary:
        print("%-12s paths %2d terms %3d" % (tag, P, T))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1] if len(sys.argv) > 1 else OUT))
