"""ORACLE (test infrastructure only).  Real spherical harmonics, real Clebsch-Gordan coefficients
and real Wigner-D matrices in float64, written from their textbook definitions.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.  It
shares no code with the HIP library: its SH come from the Cartesian real-form formula and its CG
from Racah's formula, while the library uses hand-expanded polynomials and a quadrature
construction.

The pages ("Fast and Accurate Foundation Models for Equivariant MLIPs", Sec. VII, on
parity-restricted irreps; "FlashCart", Fig. C1 / Table C1, on coupling counts ordered by
J = l1 + l2 + l3) name these objects but define none of them; the conventions below are the
plainest standard ones:
  * real SH, component normalisation (sum_m Y_lm^2 = 2l + 1, Y_0 = 1), m = -l..l, with
    Y_1 = sqrt(3) (y, z, x);
  * complex SH with the Condon-Shortley phase; real = sqrt(4 pi) Q_l complex with the unitary
    Q_l below;
  * real CG = (conj Q_l1 x conj Q_l2 x Q_l3) applied to the Condon-Shortley CG; for
    l1 + l2 + l3 even it is real and orthonormal over (m1, m2) for each m3.
"""
from __future__ import annotations

from fractions import Fraction
from functools import lru_cache
from math import comb, factorial, sqrt, pi

import numpy as np


# ----------------------------------------------------------------------------------------------
# Real spherical harmonics as homogeneous polynomials (Cartesian real form).
#
# For m > 0:  Y_lm = sqrt((2l+1)/(2 pi)) Pi_l^m(z) A_m(x, y)
# for m < 0:  Y_lm = sqrt((2l+1)/(2 pi)) Pi_l^|m|(z) B_|m|(x, y)
# for m = 0:  Y_l0 = sqrt((2l+1)/(4 pi)) Pi_l^0(z)
# with A_m + i B_m = (x + i y)^m and
# Pi_l^m(z) = sqrt((l-m)!/(l+m)!) sum_k (-1)^k 2^-l C(l,k) C(2l-2k,l) (l-2k)!/(l-2k-m)! r^2k z^(l-2k-m).
# These are orthonormal; multiplying by sqrt(4 pi) gives component normalisation.  r^2 is expanded
# as x^2 + y^2 + z^2 so that each Y_lm is a homogeneous polynomial of degree l.
# ----------------------------------------------------------------------------------------------

def _poly_mul(a: dict, b: dict) -> dict:
    out: dict = {}
    for ea, ca in a.items():
        for eb, cb in b.items():
            e = (ea[0] + eb[0], ea[1] + eb[1], ea[2] + eb[2])
            out[e] = out.get(e, 0.0) + ca * cb
    return out


def _poly_pow(a: dict, n: int) -> dict:
    out = {(0, 0, 0): 1.0}
    for _ in range(n):
        out = _poly_mul(out, a)
    return out


@lru_cache(maxsize=None)
def sh_polynomial(l: int, m: int):
    """Monomial coefficients {(a, b, c): coef} of the component-normalised real Y_lm, i.e.
    Y_lm(x, y, z) = sum coef * x^a y^b z^c for unit (x, y, z)."""
    am = abs(m)
    r2 = {(2, 0, 0): 1.0, (0, 2, 0): 1.0, (0, 0, 2): 1.0}
    pi_poly: dict = {}
    for k in range((l - am) // 2 + 1):
        c = ((-1) ** k) * 2.0 ** (-l) * comb(l, k) * comb(2 * l - 2 * k, l) \
            * factorial(l - 2 * k) / factorial(l - 2 * k - am)
        term = _poly_mul(_poly_pow(r2, k), {(0, 0, l - 2 * k - am): c})
        for e, v in term.items():
            pi_poly[e] = pi_poly.get(e, 0.0) + v
    norm_pi = sqrt(factorial(l - am) / factorial(l + am))
    # (x + i y)^m expanded: sum_p C(m,p) x^p (i y)^(m-p)
    ab: dict = {}
    for p in range(am + 1):
        ipow = (am - p) % 4            # i^(m-p) = 1, i, -1, -i
        re, im = [(1, 0), (0, 1), (-1, 0), (0, -1)][ipow]
        c = comb(am, p)
        val = re if m >= 0 else im
        if val != 0:
            ab[(p, am - p, 0)] = ab.get((p, am - p, 0), 0.0) + c * val
    if m == 0:
        pref = sqrt((2 * l + 1) / (4 * pi))
        ab = {(0, 0, 0): 1.0}
    else:
        pref = sqrt((2 * l + 1) / (2 * pi))
    poly = _poly_mul(pi_poly, ab)
    scale = sqrt(4 * pi) * pref * norm_pi
    return tuple(sorted((e, c * scale) for e, c in poly.items() if c != 0.0))


def _eval_poly(poly, v: np.ndarray) -> np.ndarray:
    x, y, z = v[..., 0], v[..., 1], v[..., 2]
    out = np.zeros(v.shape[:-1])
    for (a, b, c), coef in poly:
        out = out + coef * x ** a * y ** b * z ** c
    return out


def _eval_poly_grad(poly, v: np.ndarray) -> np.ndarray:
    x, y, z = v[..., 0], v[..., 1], v[..., 2]
    g = np.zeros(v.shape)
    for (a, b, c), coef in poly:
        if a:
            g[..., 0] += coef * a * x ** (a - 1) * y ** b * z ** c
        if b:
            g[..., 1] += coef * b * x ** a * y ** (b - 1) * z ** c
        if c:
            g[..., 2] += coef * c * x ** a * y ** b * z ** (c - 1)
    return g


def real_sh(l: int, u: np.ndarray) -> np.ndarray:
    """Y_l(u) for unit vectors u [..., 3] -> [..., 2l+1] (m = -l..l), component-normalised."""
    return np.stack([_eval_poly(sh_polynomial(l, m), u) for m in range(-l, l + 1)], -1)


def real_sh_grad(l: int, u: np.ndarray) -> np.ndarray:
    """Gradient of the degree-l homogeneous polynomial of each Y_lm at u: [..., 2l+1, 3]."""
    return np.stack([_eval_poly_grad(sh_polynomial(l, m), u) for m in range(-l, l + 1)], -2)


# ----------------------------------------------------------------------------------------------
# Complex <-> real change of basis.  Rows: real m; columns: complex mu; both -l..l.
# ----------------------------------------------------------------------------------------------

@lru_cache(maxsize=None)
def q_matrix(l: int) -> np.ndarray:
    Q = np.zeros((2 * l + 1, 2 * l + 1), dtype=np.complex128)
    s = 1.0 / sqrt(2.0)
    for m in range(-l, l + 1):
        r = m + l
        if m < 0:
            Q[r, l - abs(m)] = 1j * s
            Q[r, l + abs(m)] = -1j * ((-1) ** m) * s
        elif m == 0:
            Q[r, l] = 1.0
        else:
            Q[r, l - m] = s
            Q[r, l + m] = ((-1) ** m) * s
    return Q


# ----------------------------------------------------------------------------------------------
# Clebsch-Gordan coefficients: Racah's closed formula (Condon-Shortley phase), exact in rationals
# under the square root, then the real-basis transform.
# ----------------------------------------------------------------------------------------------

def cg_complex(j1: int, m1: int, j2: int, m2: int, J: int, M: int) -> float:
    """<j1 m1 j2 m2 | J M> for integer angular momenta (Racah)."""
    if M != m1 + m2 or not (abs(j1 - j2) <= J <= j1 + j2):
        return 0.0
    if abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0.0
    f = factorial
    pre = Fraction((2 * J + 1) * f(J + j1 - j2) * f(J - j1 + j2) * f(j1 + j2 - J), f(j1 + j2 + J + 1))
    pre *= f(J + M) * f(J - M) * f(j1 - m1) * f(j1 + m1) * f(j2 - m2) * f(j2 + m2)
    s = Fraction(0)
    for k in range(0, j1 + j2 + J + 1):
        args = [k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k]
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= f(a)
        s += Fraction((-1) ** k, den)
    sign = 1.0 if s >= 0 else -1.0
    # sqrt(pre) * s  computed as sign * sqrt(pre * s^2) to keep the rational exact until the end
    return sign * sqrt(float(pre * s * s))


@lru_cache(maxsize=None)
def real_cg(l1: int, l2: int, l3: int) -> np.ndarray:
    """C[m1, m2, m3] (shape [2l1+1, 2l2+1, 2l3+1]) in the real basis:
    sum over mu of conj(Q_l1[m1,mu1]) conj(Q_l2[m2,mu2]) Q_l3[m3,mu3] <l1 mu1 l2 mu2 | l3 mu3>."""
    cc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for a in range(-l1, l1 + 1):
        for b in range(-l2, l2 + 1):
            c = a + b
            if abs(c) <= l3:
                cc[a + l1, b + l2, c + l3] = cg_complex(l1, a, l2, b, l3, c)
    Q1, Q2, Q3 = q_matrix(l1), q_matrix(l2), q_matrix(l3)
    out = np.einsum("ai,bj,ck,ijk->abc", Q1.conj(), Q2.conj(), Q3, cc)
    if (l1 + l2 + l3) % 2 == 0:
        assert np.max(np.abs(out.imag)) < 1e-12, "real CG must be real for even l1+l2+l3"
        return np.ascontiguousarray(out.real)
    return out


# ----------------------------------------------------------------------------------------------
# Paths: ordered triples (l1 in input, l2 in SH, l3 in output) with the triangle rule and
# l1 + l2 + l3 even (parity-restricted irreps), in lexicographic order.
# ----------------------------------------------------------------------------------------------

def paths(L_in: int, L_sh: int, L_out: int):
    out = []
    for l1 in range(L_in + 1):
        for l2 in range(L_sh + 1):
            for l3 in range(L_out + 1):
                if abs(l1 - l2) <= l3 <= l1 + l2 and (l1 + l2 + l3) % 2 == 0:
                    out.append((l1, l2, l3))
    return out


# ----------------------------------------------------------------------------------------------
# Wigner-D: Wigner's small-d formula, complex D for the active rotation R = Rz(a) Ry(b) Rz(c),
# then the real basis.  With Y(R u) = conj(D(R)) Y(u) for complex SH, the real matrix is
# D_real = Q conj(D) Q^H, so that Y_real(R u) = D_real(R) Y_real(u).
# ----------------------------------------------------------------------------------------------

def rotation_zyz(a: float, b: float, c: float) -> np.ndarray:
    def rz(t):
        return np.array([[np.cos(t), -np.sin(t), 0], [np.sin(t), np.cos(t), 0], [0, 0, 1.0]])

    def ry(t):
        return np.array([[np.cos(t), 0, np.sin(t)], [0, 1.0, 0], [-np.sin(t), 0, np.cos(t)]])
    return rz(a) @ ry(b) @ rz(c)


def wigner_small_d(l: int, b: float) -> np.ndarray:
    d = np.zeros((2 * l + 1, 2 * l + 1))
    cb, sb = np.cos(b / 2), np.sin(b / 2)
    f = factorial
    for mp in range(-l, l + 1):
        for m in range(-l, l + 1):
            pre = sqrt(f(l + mp) * f(l - mp) * f(l + m) * f(l - m))
            s = 0.0
            for k in range(0, 2 * l + 1):
                a1, a2, a3, a4 = l + m - k, k, mp - m + k, l - mp - k
                if min(a1, a2, a3, a4) < 0:
                    continue
                s += ((-1) ** (mp - m + k)) / (f(a1) * f(a2) * f(a3) * f(a4)) \
                    * cb ** (2 * l + m - mp - 2 * k) * sb ** (mp - m + 2 * k)
            d[mp + l, m + l] = pre * s
    return d


def wigner_d_real(l: int, a: float, b: float, c: float) -> np.ndarray:
    ms = np.arange(-l, l + 1)
    D = np.exp(-1j * ms[:, None] * a) * wigner_small_d(l, b) * np.exp(-1j * ms[None, :] * c)
    Q = q_matrix(l)
    out = Q @ D.conj() @ Q.conj().T
    assert np.max(np.abs(out.imag)) < 1e-12
    return np.ascontiguousarray(out.real)
