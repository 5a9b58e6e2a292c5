"""Real Clebsch-Gordan tensors and real Wigner D matrices (test infrastructure).

The e3nn_mlx README (feature list) promises e3nn-compatible real Wigner-3j /
Clebsch-Gordan coefficients and real Wigner matrices with O(3) parity; no
formula or fixture is printed on the pages, so this module derives them from
the textbook definitions:

* complex CG coefficients from Racah's closed formula (exact rational
  arithmetic for everything under the square root and in the alternating sum);
* the unitary map from Condon-Shortley complex spherical harmonics to real
  ones (m = -l..l, z polar axis, so l=1 components are ordered (y, z, x));
* the real CG tensor ``C[m1, m2, m3]`` as the complex CG conjugated into the
  real basis, made real by one global phase, with the sign chosen so that the
  first nonzero entry in (m1, m2, m3) array order is positive.  No extra
  factor is applied: the Racah coefficients already satisfy
  ``sum_{m1,m2} C[m1,m2,m3] C[m1,m2,m3'] = delta``, which is the reading used
  for the e3j ``SQRT_DIM_OUT`` tensor-product normalization (the e3j
  Convolution page names it without giving a formula);
* real Wigner D matrices as the exponential map of the angular-momentum
  generators, conjugated into the same real basis, so that real spherical
  harmonics satisfy ``Y(R v) = D(R) Y(v)``; inversion acts as ``p`` on an
  irrep of parity ``p`` (e3nn_mlx README, O(3) parity transforms).

Everything here is fp64 / complex128 numpy.  Pinned by tests/test_oracle_so3.py.
"""

import math
from fractions import Fraction
from functools import lru_cache

import numpy as np
from scipy.linalg import expm


def _fact(n):
    return math.factorial(n)


def racah_cg(j1, m1, j2, m2, J, M):
    """Complex (Condon-Shortley) CG coefficient <j1 m1 j2 m2 | J M>, integer spins.

    Racah's formula: a square-root prefactor of factorials times an
    alternating sum over k of 1/(products of six factorials); k runs over all
    integers keeping every factorial argument non-negative.
    """
    if M != m1 + m2:
        return 0.0
    if not (abs(j1 - j2) <= J <= j1 + j2):
        return 0.0
    if abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0.0
    pre = Fraction(
        (2 * J + 1) * _fact(j1 + j2 - J) * _fact(j1 - j2 + J) * _fact(-j1 + j2 + J),
        _fact(j1 + j2 + J + 1),
    )
    pre *= (
        _fact(j1 + m1) * _fact(j1 - m1) * _fact(j2 + m2) * _fact(j2 - m2)
        * _fact(J + M) * _fact(J - M)
    )
    total = Fraction(0)
    for k in range(0, j1 + j2 + J + 2):
        args = (k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k,
                J - j2 + m1 + k, J - j1 - m2 + k)
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= _fact(a)
        total += Fraction((-1) ** k, den)
    return float(total) * math.sqrt(float(pre))


@lru_cache(maxsize=None)
def complex_cg(l1, l2, l3):
    """Array CG[mu1, mu2, mu3] over mu = -l..l (index mu + l)."""
    out = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for a in range(-l1, l1 + 1):
        for b in range(-l2, l2 + 1):
            c = a + b
            if abs(c) <= l3:
                out[a + l1, b + l2, c + l3] = racah_cg(l1, a, l2, b, l3, c)
    out.setflags(write=False)
    return out


@lru_cache(maxsize=None)
def real_basis(l):
    """Unitary U with Y_real = U @ Y_complex (Condon-Shortley complex harmonics).

    Rows are real components m = -l..l, columns complex components mu = -l..l:
      m > 0 : (-1)^m / sqrt2 on mu = m,  1 / sqrt2 on mu = -m
      m = 0 : 1 on mu = 0
      m < 0 : i / sqrt2 on mu = m,  -i (-1)^|m| / sqrt2 on mu = |m|
    """
    U = np.zeros((2 * l + 1, 2 * l + 1), dtype=complex)
    r = 1 / math.sqrt(2)
    for m in range(-l, l + 1):
        i = m + l
        if m > 0:
            U[i, m + l] = (-1) ** m * r
            U[i, -m + l] = r
        elif m == 0:
            U[i, l] = 1.0
        else:
            am = -m
            U[i, m + l] = 1j * r
            U[i, am + l] = -1j * (-1) ** am * r
    U.setflags(write=False)
    return U


@lru_cache(maxsize=None)
def real_cg(l1, l2, l3):
    """Real CG tensor C[m1, m2, m3] (shape (2l1+1, 2l2+1, 2l3+1)).

    out_real[m3] = sum_{m1,m2} C[m1,m2,m3] x_real[m1] y_real[m2] couples two
    real-basis irreps into l3.  Returns zeros if the triangle rule fails.
    """
    if not (abs(l1 - l2) <= l3 <= l1 + l2):
        z = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
        z.setflags(write=False)
        return z
    U1, U2, U3 = real_basis(l1), real_basis(l2), real_basis(l3)
    cg = complex_cg(l1, l2, l3)
    # x_c = U1^H x_r, y_c = U2^H y_r, out_r = U3 out_c
    T = np.einsum("kc,abc,ia,jb->ijk", U3, cg, U1.conj(), U2.conj())
    flat = T.reshape(-1)
    big = flat[np.argmax(np.abs(flat))]
    T = T / (big / abs(big))
    scale = np.abs(T).max()
    if np.abs(T.imag).max() > 1e-12 * scale:
        raise AssertionError(f"real CG ({l1},{l2},{l3}) is not real after phase fix")
    T = T.real.copy()
    T[np.abs(T) < 1e-14 * scale] = 0.0
    nz = np.flatnonzero(T.reshape(-1))
    if T.reshape(-1)[nz[0]] < 0:
        T = -T
    T.setflags(write=False)
    return T


# ---------------------------------------------------------------- Wigner D ---

@lru_cache(maxsize=None)
def _complex_generators(l):
    """Complex angular-momentum matrices (Jx, Jy, Jz) in the |l mu> basis."""
    n = 2 * l + 1
    Jz = np.diag(np.arange(-l, l + 1).astype(complex))
    Jp = np.zeros((n, n), dtype=complex)
    for mu in range(-l, l):
        Jp[mu + 1 + l, mu + l] = math.sqrt(l * (l + 1) - mu * (mu + 1))
    Jm = Jp.conj().T
    Jx = (Jp + Jm) / 2
    Jy = (Jp - Jm) / (2j)
    return Jx, Jy, Jz


@lru_cache(maxsize=None)
def real_generators(l):
    """Real antisymmetric generators (Gx, Gy, Gz) with D(exp(theta n.L)) = expm(theta n.G).

    The complex rotation operator about unit axis n is expm(-i theta n.J);
    harmonics transform with its complex conjugate, Y(Rv) = conj(D_c) Y(v),
    which in the real basis is expm(theta * n.G) with G = U conj(-i J) U^H.
    """
    U = real_basis(l)
    gens = []
    for J in _complex_generators(l):
        G = U @ np.conj(-1j * J) @ U.conj().T
        if np.abs(G.imag).max() > 1e-12:
            raise AssertionError("real generator is not real")
        gens.append(G.real.copy())
    return tuple(gens)


def rotation_matrix(axis, angle):
    """3x3 rotation about ``axis`` by ``angle`` (Rodrigues' formula)."""
    n = np.asarray(axis, dtype=float)
    n = n / np.linalg.norm(n)
    K = np.array([[0, -n[2], n[1]], [n[2], 0, -n[0]], [-n[1], n[0], 0]])
    return np.eye(3) + math.sin(angle) * K + (1 - math.cos(angle)) * (K @ K)


def wigner_D(l, axis, angle, parity=1, improper=False):
    """Real Wigner D of the O(3) element g = (+/-) R(axis, angle) on irrep (l, parity).

    For the proper part: D = expm(angle * n.G).  ``improper=True`` means
    g = -R, which multiplies the matrix by ``parity``.
    """
    n = np.asarray(axis, dtype=float)
    n = n / np.linalg.norm(n)
    Gx, Gy, Gz = real_generators(l)
    D = expm(angle * (n[0] * Gx + n[1] * Gy + n[2] * Gz))
    if improper:
        D = parity * D
    return D


def block_D(blocks, axis, angle, improper=False):
    """Block-diagonal D over a list of (mul, l, parity) blocks (per channel)."""
    mats = [wigner_D(l, axis, angle, p, improper) for (_, l, p) in blocks]
    n = sum(m.shape[0] for m in mats)
    out = np.zeros((n, n))
    o = 0
    for m in mats:
        k = m.shape[0]
        out[o:o + k, o:o + k] = m
        o += k
    return out
