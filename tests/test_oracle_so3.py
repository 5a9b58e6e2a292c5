"""Pins for the oracle's SO(3)/O(3) tables and the generator's spherical harmonics.

Each pin ties a function to something other than itself: a library routine
(sympy's Clebsch-Gordan, scipy's Legendre polynomials), a textbook closed form,
a group-theoretic identity, or hand-derived golden values.
"""

import math

import numpy as np
import pytest
from scipy.special import eval_legendre

from oracle import so3
from equivariant_gnn_message_amd import synth

from ._util import eval_array, load_golden, random_rotation

LMAX = 4


def triples(lmax=LMAX):
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax + 2) + 1):
                yield l1, l2, l3


# ------------------------------------------------------------ complex CG ---

def test_racah_matches_sympy():
    """Racah closed form against sympy's independent Clebsch-Gordan routine."""
    from sympy.physics.quantum.cg import CG
    for l1 in range(4):
        for l2 in range(4):
            for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                for m1 in range(-l1, l1 + 1):
                    for m2 in range(-l2, l2 + 1):
                        m3 = m1 + m2
                        if abs(m3) > l3:
                            continue
                        ref = float(CG(l1, m1, l2, m2, l3, m3).doit().evalf(30))
                        got = so3.racah_cg(l1, m1, l2, m2, l3, m3)
                        assert abs(got - ref) < 1e-13, (l1, m1, l2, m2, l3, m3, got, ref)


def test_racah_textbook_values():
    r = so3.racah_cg
    assert abs(r(1, 1, 1, -1, 0, 0) - 1 / math.sqrt(3)) < 1e-15
    assert abs(r(1, 0, 1, 0, 0, 0) + 1 / math.sqrt(3)) < 1e-15
    assert abs(r(1, 0, 1, 0, 2, 0) - math.sqrt(2 / 3)) < 1e-15
    assert r(1, 0, 1, 0, 1, 0) == 0.0
    assert abs(r(1, 1, 1, -1, 1, 0) - 1 / math.sqrt(2)) < 1e-15
    assert abs(r(2, 2, 2, -2, 0, 0) - 1 / math.sqrt(5)) < 1e-15
    assert r(1, 1, 1, 1, 1, 1) == 0.0   # M != m1 + m2 is excluded below
    assert r(1, 1, 1, 0, 1, 0) == 0.0


# --------------------------------------------------------------- real CG ---

@pytest.mark.parametrize("l1,l2,l3", list(triples()))
def test_real_cg_orthonormal(l1, l2, l3):
    C = so3.real_cg(l1, l2, l3)
    if not (abs(l1 - l2) <= l3 <= l1 + l2):
        assert not C.any()
        return
    G = np.einsum("abk,abq->kq", C, C)
    np.testing.assert_allclose(G, np.eye(2 * l3 + 1), atol=1e-13)


@pytest.mark.parametrize("l1,l2", [(a, b) for a in range(LMAX + 1) for b in range(LMAX + 1)])
def test_real_cg_complete(l1, l2):
    """sum over l3, m3 of C C = identity on (m1, m2): no coupling is missing."""
    n1, n2 = 2 * l1 + 1, 2 * l2 + 1
    S = np.zeros((n1 * n2, n1 * n2))
    for l3 in range(abs(l1 - l2), l1 + l2 + 1):
        C = so3.real_cg(l1, l2, l3).reshape(n1 * n2, -1)
        S += C @ C.T
    np.testing.assert_allclose(S, np.eye(n1 * n2), atol=1e-13)


@pytest.mark.parametrize("l1,l2,l3", [t for t in triples() if abs(t[0] - t[1]) <= t[2] <= t[0] + t[1]])
def test_real_cg_invariant(l1, l2, l3):
    rng = np.random.default_rng(100 + 16 * l1 + 4 * l2 + l3)
    for _ in range(2):
        axis, ang = random_rotation(rng)
        D1, D2, D3 = (so3.wigner_D(l, axis, ang) for l in (l1, l2, l3))
        C = so3.real_cg(l1, l2, l3)
        rot = np.einsum("ai,bj,ck,ijk->abc", D1, D2, D3, C)
        np.testing.assert_allclose(rot, C, atol=1e-12)


@pytest.mark.parametrize("l1,l2,l3", [t for t in triples() if abs(t[0] - t[1]) <= t[2] <= t[0] + t[1]])
def test_real_cg_selection_rule(l1, l2, l3):
    """Nonzero only if |m3| in {|m1|+|m2|, ||m1|-|m2||} and #(m<0) = l1+l2+l3 mod 2."""
    C = so3.real_cg(l1, l2, l3)
    for i, j, k in zip(*np.nonzero(C)):
        m1, m2, m3 = int(i) - l1, int(j) - l2, int(k) - l3
        assert abs(m3) in (abs(m1) + abs(m2), abs(abs(m1) - abs(m2)))
        neg = int(m1 < 0) + int(m2 < 0) + int(m3 < 0)
        assert neg % 2 == (l1 + l2 + l3) % 2


def test_real_cg_closed_forms():
    s2, s3 = math.sqrt(2), math.sqrt(3)
    for l in range(5):
        np.testing.assert_allclose(so3.real_cg(0, l, l)[0], np.eye(2 * l + 1), atol=1e-15)
        np.testing.assert_allclose(so3.real_cg(l, 0, l)[:, 0, :], np.eye(2 * l + 1), atol=1e-15)
    np.testing.assert_allclose(so3.real_cg(1, 1, 0)[:, :, 0], np.eye(3) / s3, atol=1e-15)
    eps = np.zeros((3, 3, 3))
    for (i, j, k) in [(0, 1, 2), (1, 2, 0), (2, 0, 1)]:
        eps[i, j, k] = 1.0
        eps[j, i, k] = -1.0
    np.testing.assert_allclose(so3.real_cg(1, 1, 1), eps / s2, atol=1e-15)


def test_real_cg_sign_rule():
    for l1, l2, l3 in triples():
        C = so3.real_cg(l1, l2, l3)
        nz = np.flatnonzero(C.reshape(-1))
        if len(nz):
            assert C.reshape(-1)[nz[0]] > 0


def test_nonzero_counts_of_workload_layouts():
    """Sum of nonzero CG entries per layout (37/58/86/215 for the four layouts)."""
    from oracle import conv
    expect = {0: 37, 1: 58, 2: 86, 3: 215}
    for idx, nnz in expect.items():
        w = synth.WORKLOADS[idx]
        lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
        got = sum(int(np.count_nonzero(so3.real_cg(p.l1, p.l2, p.l3))) for p in lay.paths)
        assert got == nnz, (idx, got)


# --------------------------------------------------------------- Wigner D ---

def test_wigner_D_l1_is_permuted_rotation():
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)   # (x,y,z) -> (y,z,x)
    rng = np.random.default_rng(1)
    for _ in range(5):
        axis, ang = random_rotation(rng)
        R = so3.rotation_matrix(axis, ang)
        np.testing.assert_allclose(so3.wigner_D(1, axis, ang), P @ R @ P.T, atol=1e-14)


def test_rotation_matrix_is_rotation():
    rng = np.random.default_rng(2)
    axis, ang = random_rotation(rng)
    R = so3.rotation_matrix(axis, ang)
    np.testing.assert_allclose(R @ R.T, np.eye(3), atol=1e-15)
    assert abs(np.linalg.det(R) - 1) < 1e-14
    np.testing.assert_allclose(R @ axis, axis, atol=1e-15)


@pytest.mark.parametrize("l", range(6))
def test_wigner_D_orthogonal_and_homomorphism(l):
    from scipy.spatial.transform import Rotation
    rng = np.random.default_rng(10 + l)
    a1, t1 = random_rotation(rng)
    a2, t2 = random_rotation(rng)
    D1 = so3.wigner_D(l, a1, t1)
    D2 = so3.wigner_D(l, a2, t2)
    np.testing.assert_allclose(D1 @ D1.T, np.eye(2 * l + 1), atol=1e-13)
    R12 = so3.rotation_matrix(a1, t1) @ so3.rotation_matrix(a2, t2)
    rv = Rotation.from_matrix(R12).as_rotvec()
    ang = np.linalg.norm(rv)
    D12 = so3.wigner_D(l, rv / ang, ang)
    np.testing.assert_allclose(D12, D1 @ D2, atol=1e-12)


@pytest.mark.parametrize("l,p", [(l, p) for l in range(4) for p in (1, -1)])
def test_wigner_D_inversion(l, p):
    D = so3.wigner_D(l, [0, 0, 1], 0.0, parity=p, improper=True)
    np.testing.assert_allclose(D, p * np.eye(2 * l + 1), atol=1e-15)


# ----------------------------------------------------- spherical harmonics ---

def test_sh_golden_values():
    gold = load_golden("sh_closed_forms.json")
    v = eval_array(gold["vector"])
    Y = synth.spherical_harmonics(3, v[None, :])[0]
    for l in range(4):
        np.testing.assert_allclose(Y[l * l:(l + 1) ** 2], eval_array(gold["values"][str(l)]), atol=1e-14)


def test_sh_addition_theorem():
    rng = np.random.default_rng(3)
    u = rng.standard_normal((50, 3))
    v = rng.standard_normal((50, 3))
    Yu = synth.spherical_harmonics(3, u)
    Yv = synth.spherical_harmonics(3, v)
    cos = np.sum(u * v, 1) / np.linalg.norm(u, axis=1) / np.linalg.norm(v, axis=1)
    for l in range(4):
        lhs = np.sum(Yu[:, l * l:(l + 1) ** 2] * Yv[:, l * l:(l + 1) ** 2], 1)
        np.testing.assert_allclose(lhs, (2 * l + 1) * eval_legendre(l, cos), atol=1e-12)


def test_sh_parity_and_norm():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((20, 3))
    Y = synth.spherical_harmonics(3, v)
    Ym = synth.spherical_harmonics(3, -v)
    for l in range(4):
        sl = slice(l * l, (l + 1) ** 2)
        np.testing.assert_allclose(Ym[:, sl], (-1) ** l * Y[:, sl], atol=1e-13)
        np.testing.assert_allclose(np.sum(Y[:, sl] ** 2, 1), 2 * l + 1, atol=1e-12)


def test_sh_equivariant_under_oracle_D():
    """Y(R v) = D(R) Y(v): ties the generator's harmonics to the oracle's basis."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((10, 3))
    for _ in range(3):
        axis, ang = random_rotation(rng)
        R = so3.rotation_matrix(axis, ang)
        Y = synth.spherical_harmonics(3, v)
        YR = synth.spherical_harmonics(3, v @ R.T)
        for l in range(4):
            sl = slice(l * l, (l + 1) ** 2)
            np.testing.assert_allclose(YR[:, sl], Y[:, sl] @ so3.wigner_D(l, axis, ang).T, atol=1e-12)


def test_sh_recursion_equals_closed_forms():
    """The associated-Legendre recursion reproduces the hand-written l <= 3 forms."""
    v = np.random.default_rng(6).standard_normal((40, 3))
    np.testing.assert_allclose(synth.sh_by_recursion(3, v), synth.spherical_harmonics(3, v), atol=1e-14)


@pytest.mark.parametrize("lmax", [6, 8])
def test_sh_high_l_addition_parity_norm(lmax):
    """Up to l = 8: the addition theorem against scipy's Legendre polynomials, parity
    (-1)^l under v -> -v, and the component norm 2l+1."""
    rng = np.random.default_rng(lmax)
    u = rng.standard_normal((60, 3))
    v = rng.standard_normal((60, 3))
    Yu = synth.spherical_harmonics(lmax, u)
    Yv = synth.spherical_harmonics(lmax, v)
    Ym = synth.spherical_harmonics(lmax, -v)
    assert Yu.shape == (60, (lmax + 1) ** 2)
    cos = np.sum(u * v, 1) / np.linalg.norm(u, axis=1) / np.linalg.norm(v, axis=1)
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        np.testing.assert_allclose(np.sum(Yu[:, sl] * Yv[:, sl], 1), (2 * l + 1) * eval_legendre(l, cos),
                                   atol=1e-10)
        np.testing.assert_allclose(Ym[:, sl], (-1) ** l * Yv[:, sl], atol=1e-12)
        np.testing.assert_allclose(np.sum(Yv[:, sl] ** 2, 1), 2 * l + 1, atol=1e-10)


def test_sh_high_l_equivariant_under_oracle_D():
    """Y(R v) = D(R) Y(v) for l = 4..6 with the oracle's Wigner D (the basis and the m
    order of the recursion agree with the oracle's real basis)."""
    rng = np.random.default_rng(9)
    v = rng.standard_normal((8, 3))
    axis, ang = random_rotation(rng)
    R = so3.rotation_matrix(axis, ang)
    Y = synth.spherical_harmonics(6, v)
    YR = synth.spherical_harmonics(6, v @ R.T)
    for l in range(4, 7):
        sl = slice(l * l, (l + 1) ** 2)
        np.testing.assert_allclose(YR[:, sl], Y[:, sl] @ so3.wigner_D(l, axis, ang).T, atol=1e-10)


def test_sh_shapes():
    v = np.ones((2, 3))
    Y = synth.spherical_harmonics(2, v)
    assert Y.shape == (2, 9)
    blocks = {l: Y[:, l * l:(l + 1) ** 2].shape for l in range(3)}
    assert blocks == {0: (2, 1), 1: (2, 3), 2: (2, 5)}
