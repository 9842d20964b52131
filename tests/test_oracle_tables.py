"""Pins of the oracle's Clebsch-Gordan tables, spherical harmonics and Wigner-D.

Everything here is fixed by mathematics or an independent library routine, not by
the oracle itself: sympy's exact CG values, closed forms, orthogonality, the
rotation group law and the transformation law of spherical harmonics.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import sphere

TRIPLES = [(l1, l2, l3) for l1 in range(4) for l2 in range(4) for l3 in range(4)
           if abs(l1 - l2) <= l3 <= l1 + l2]


def test_cg_check_value():
    assert oracle.cg_complex(1, 1, 1, -1, 0, 0) == pytest.approx(1 / math.sqrt(3), abs=1e-15)


def test_cg_complex_matches_sympy():
    from sympy import S
    from sympy.physics.quantum.cg import CG
    worst = 0.0
    for j1, j2, J in TRIPLES:
        for m1 in range(-j1, j1 + 1):
            for m2 in range(-j2, j2 + 1):
                M = m1 + m2
                if abs(M) > J:
                    assert oracle.cg_complex(j1, m1, j2, m2, J, M) == 0.0
                    continue
                ref = float(CG(S(j1), S(m1), S(j2), S(m2), S(J), S(M)).doit())
                got = oracle.cg_complex(j1, m1, j2, m2, J, M)
                worst = max(worst, abs(ref - got))
    assert worst < 1e-14
    # selection rules: M = m1 + m2 and the triangle rule
    assert oracle.cg_complex(1, 0, 1, 0, 1, 1) == 0.0
    assert oracle.cg_complex(1, 0, 1, 0, 3, 0) == 0.0
    # <1 0 1 0|1 0> vanishes (the antisymmetric l=1 coupling has no m=0 x m=0 term)
    assert abs(oracle.cg_complex(1, 0, 1, 0, 1, 0)) < 1e-16


def test_complex_cg_orthogonality():
    for j1, j2 in itertools.product(range(4), range(4)):
        Js = range(abs(j1 - j2), j1 + j2 + 1)
        for J, Jp in itertools.product(Js, Js):
            for M in range(-J, J + 1):
                for Mp in range(-Jp, Jp + 1):
                    s = sum(oracle.cg_complex(j1, m1, j2, m2, J, M) *
                            oracle.cg_complex(j1, m1, j2, m2, Jp, Mp)
                            for m1 in range(-j1, j1 + 1) for m2 in range(-j2, j2 + 1))
                    assert abs(s - (1.0 if (J, M) == (Jp, Mp) else 0.0)) < 1e-13


def test_real_basis_is_unitary():
    for l in range(4):
        A = oracle.real_basis(l)
        assert np.allclose(A @ A.conj().T, np.eye(2 * l + 1), atol=1e-15)


@pytest.mark.parametrize("l1,l2,l3", TRIPLES)
def test_real_cg_realness_by_parity(l1, l2, l3):
    T = oracle.cg_real_raw(l1, l2, l3)
    if (l1 + l2 + l3) % 2 == 0:
        assert np.abs(T.imag).max() < 1e-13
        assert np.abs(T.real).max() > 0.1
    else:
        assert np.abs(T.real).max() < 1e-13
        assert np.abs(T.imag).max() > 0.1


@pytest.mark.parametrize("l1,l2,l3", TRIPLES)
def test_real_cg_orthonormal_and_canonical(l1, l2, l3):
    C = oracle.cg_real(l1, l2, l3)
    n3 = 2 * l3 + 1
    G = C.reshape(-1, n3).T @ C.reshape(-1, n3)
    assert np.allclose(G, np.eye(n3), atol=1e-13)
    flat = C.ravel()
    first = flat[np.nonzero(np.abs(flat) > 1e-10)[0][0]]
    assert first > 0
    nz = flat[flat != 0]
    assert np.abs(nz).min() > 0.1          # structural zeros are exact zeros


def test_real_cg_out_of_triangle_is_zero():
    assert not oracle.cg_real(1, 1, 3).any()
    assert not oracle.cg_real(0, 2, 1).any()


def test_real_cg_closed_forms():
    for l in range(4):
        n = 2 * l + 1
        assert np.allclose(oracle.cg_real(l, 0, l)[:, 0, :], np.eye(n), atol=1e-14)
        assert np.allclose(oracle.cg_real(0, l, l)[0, :, :], np.eye(n), atol=1e-14)
        assert np.allclose(oracle.cg_real(l, l, 0)[:, :, 0], np.eye(n) / math.sqrt(n), atol=1e-14)
    # 1 x 1 -> 1 is the cross product; in the (y, z, x) order the Levi-Civita
    # symbol over (y, z, x) indices is a cyclic relabelling of the xyz one.
    eps = np.zeros((3, 3, 3))
    for (a, b, c), s in {(0, 1, 2): 1, (1, 2, 0): 1, (2, 0, 1): 1,
                         (0, 2, 1): -1, (2, 1, 0): -1, (1, 0, 2): -1}.items():
        eps[a, b, c] = s
    C111 = oracle.cg_real(1, 1, 1)
    assert np.allclose(C111, eps / math.sqrt(2), atol=1e-14)
    # 1 x 1 -> 2, m3 = 0 (the 3z^2 - r^2 component): diag(1, -2, 1)/sqrt(6) in (y, z, x)
    C112 = oracle.cg_real(1, 1, 2)
    assert np.allclose(C112[:, :, 2], np.diag([1.0, -2.0, 1.0]) / math.sqrt(6), atol=1e-14)


def test_real_cg_nonzero_counts():
    expect = {(1, 1, 1): 6, (1, 1, 2): 11, (1, 2, 2): 16, (1, 2, 3): 21, (1, 3, 3): 26,
              (2, 2, 2): 25, (2, 2, 3): 28, (2, 3, 3): 41}
    for k, v in expect.items():
        assert np.count_nonzero(oracle.cg_real(*k)) == v
    for l in range(4):
        for t in [(0, l, l), (l, 0, l), (l, l, 0)]:
            assert np.count_nonzero(oracle.cg_real(*t)) == 2 * l + 1


@pytest.mark.parametrize("l1,l2,l3", TRIPLES)
def test_real_cg_intertwines_rotations(l1, l2, l3):
    """sum C[a,b,c] D1[a,i] D2[b,j] = sum D3[c,k] C[i,j,k]: the table commutes
    with rotations, which is what makes the product equivariant."""
    C = oracle.cg_real(l1, l2, l3)
    ang = (0.4, 1.3, -2.2)
    D1, D2, D3 = (sphere.wigner_d_real(l, *ang) for l in (l1, l2, l3))
    # C(D1 x, D2 y) = D3 C(x, y)  <=>  sum_ab C[a,b,c] D1[a,i] D2[b,j] = sum_k D3[c,k] C[i,j,k]
    lhs = np.einsum("abc,ai,bj->ijc", C, D1, D2)
    rhs = np.einsum("ck,ijk->ijc", D3, C)
    assert np.allclose(lhs, rhs, atol=1e-12)


# ---------------------------------------------------------------------------
# Spherical harmonics and Wigner-D (test utilities, pinned here)
# ---------------------------------------------------------------------------

def test_generator_sh_matches_legendre_construction():
    v = synth.unit_vectors(200, np.random.default_rng(3))
    assert np.allclose(synth.real_sh_cartesian(3, v), sphere.sh_real(3, v), atol=1e-13)


def test_sh_l1_is_scaled_yzx():
    v = synth.unit_vectors(50, np.random.default_rng(4))
    Y = sphere.sh_real(1, v)
    assert np.allclose(Y[:, 0], 1.0)
    assert np.allclose(Y[:, 1:4], math.sqrt(3) * v[:, [1, 2, 0]], atol=1e-14)


def test_sh_addition_theorem():
    v = synth.unit_vectors(100, np.random.default_rng(5))
    Y = sphere.sh_real(3, v)
    for l in range(4):
        assert np.allclose((Y[:, l * l:(l + 1) ** 2] ** 2).sum(1), 2 * l + 1, atol=1e-12)


def test_sh_orthonormal_by_quadrature():
    t, wt = np.polynomial.legendre.leggauss(8)
    nphi = 16
    phi = 2 * np.pi * np.arange(nphi) / nphi
    T, PHI = np.meshgrid(t, phi, indexing="ij")
    st = np.sqrt(1 - T ** 2)
    vec = np.stack([st * np.cos(PHI), st * np.sin(PHI), T], -1).reshape(-1, 3)
    w = (wt[:, None] * np.full(nphi, 2 * np.pi / nphi)[None, :]).reshape(-1)
    Y = synth.real_sh_cartesian(3, vec)
    G = (Y * w[:, None]).T @ Y / (4 * np.pi)
    assert np.allclose(G, np.eye(16), atol=1e-13)


def _euler_zyz(R):
    b = math.acos(max(-1.0, min(1.0, R[2, 2])))
    if abs(math.sin(b)) < 1e-9:
        return math.atan2(R[1, 0], R[0, 0]), b, 0.0
    a = math.atan2(R[1, 2], R[0, 2])
    c = math.atan2(R[2, 1], -R[2, 0])
    return a, b, c


def test_wigner_identity_orthogonal_and_group_law():
    rng = np.random.default_rng(6)
    for l in range(4):
        assert np.allclose(sphere.wigner_d_real(l, 0, 0, 0), np.eye(2 * l + 1), atol=1e-14)
    for _ in range(3):
        a1, a2 = rng.uniform(-3, 3, 3), rng.uniform(-3, 3, 3)
        a1[1], a2[1] = abs(a1[1]) % math.pi, abs(a2[1]) % math.pi
        R12 = sphere.rotation(*a1) @ sphere.rotation(*a2)
        e12 = _euler_zyz(R12)
        assert np.allclose(sphere.rotation(*e12), R12, atol=1e-12)
        for l in range(4):
            D1, D2 = sphere.wigner_d_real(l, *a1), sphere.wigner_d_real(l, *a2)
            assert np.allclose(D1.T @ D1, np.eye(2 * l + 1), atol=1e-12)
            assert np.allclose(D1 @ D2, sphere.wigner_d_real(l, *e12), atol=1e-11)


def test_wigner_l1_is_permuted_rotation():
    ang = (0.7, 2.0, -1.1)
    R = sphere.rotation(*ang)
    P = np.zeros((3, 3))
    P[0, 1] = P[1, 2] = P[2, 0] = 1.0        # (x, y, z) -> (y, z, x)
    assert np.allclose(sphere.wigner_d_real(1, *ang), P @ R @ P.T, atol=1e-13)


def test_sh_transform_law():
    v = synth.unit_vectors(40, np.random.default_rng(7))
    ang = (-0.9, 0.6, 2.4)
    R = sphere.rotation(*ang)
    Yn, YRn = synth.real_sh_cartesian(3, v), synth.real_sh_cartesian(3, v @ R.T)
    for l in range(4):
        D = sphere.wigner_d_real(l, *ang)
        sl = slice(l * l, (l + 1) ** 2)
        assert np.allclose(YRn[:, sl], Yn[:, sl] @ D.T, atol=1e-12)
