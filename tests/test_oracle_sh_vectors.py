"""Pins of the oracle's spherical harmonics of edge vectors and their gradient
with respect to the vector (the step before the tensor product: Y computed from
the edge vectors, and the Y gradient carried back to them).

The gradient (oracle/sphere.py, chain rule through the polar angles) is checked
against what the mathematics fixes: five-point finite differences of the values,
invariance under scaling (v . grad Y = 0, grad Y(c v) = grad Y(v) / c), the
closed form of degree 1, and rotation equivariance through the real Wigner-D."""
import math

import numpy as np
import pytest

from oracle import sphere


def _vectors(n, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, 3)) * rng.uniform(0.2, 4.0, (n, 1))


def test_values_depend_on_direction_only_and_zero_vector():
    v = _vectors(40, 1)
    n = v / np.linalg.norm(v, axis=1, keepdims=True)
    assert np.allclose(sphere.sh_of_vectors(3, v), sphere.sh_real(3, n), atol=1e-14)
    assert np.allclose(sphere.sh_of_vectors(3, 7.5 * v), sphere.sh_of_vectors(3, v), atol=1e-13)
    Y0 = sphere.sh_of_vectors(3, np.zeros((2, 3)))
    assert np.allclose(Y0, np.tile(np.eye(16)[0], (2, 1)), rtol=0, atol=1e-15)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_gradient_matches_five_point_differences(L):
    v = _vectors(60, 2)
    G = sphere.sh_grad_of_vectors(L, v)
    r = np.linalg.norm(v, axis=1, keepdims=True)
    h = 1e-3 * r                                   # a step relative to each vector's length
    for k in range(3):
        d = np.zeros((1, 3))
        d[0, k] = 1.0
        f = [sphere.sh_of_vectors(L, v + t * h * d) for t in (-2, -1, 1, 2)]
        fd = (f[0] - 8 * f[1] + 8 * f[2] - f[3]) / (12 * h)
        # truncation error of the 5-point rule: O((h/r)^4) relative to |grad Y| ~ 1/r
        assert np.abs((fd - G[:, :, k]) * r).max() < 1e-9, k


def test_gradient_scaling_laws():
    v = _vectors(50, 3)
    G = sphere.sh_grad_of_vectors(3, v)
    assert np.abs(np.einsum("emk,ek->em", G, v)).max() < 1e-13       # degree-0 homogeneity
    assert np.allclose(sphere.sh_grad_of_vectors(3, 2.5 * v), G / 2.5, atol=1e-14)
    assert not G[:, 0, :].any()                                        # Y_00 is constant
    assert not sphere.sh_grad_of_vectors(3, np.zeros((1, 3))).any()    # zero vector: zero by convention


def test_gradient_degree_one_closed_form():
    # Y_1 = sqrt(3) (y, z, x) / r, so grad of sqrt(3) c_k / r = sqrt(3) (e_k - n_k n) / r
    v = _vectors(30, 4)
    r = np.linalg.norm(v, axis=1)
    n = v / r[:, None]
    G = sphere.sh_grad_of_vectors(1, v)
    for row, k in zip((1, 2, 3), (1, 2, 0)):
        e = np.zeros(3)
        e[k] = 1.0
        want = math.sqrt(3.0) * (e[None, :] - n[:, k:k + 1] * n) / r[:, None]
        assert np.allclose(G[:, row, :], want, atol=1e-13)


def test_gradient_rotation_equivariance():
    # Y(R v) = D(R) Y(v)  =>  grad Y(R v) = D(R) grad Y(v) R^T
    v = _vectors(25, 5)
    ang = (0.7, 1.1, -0.4)
    R = sphere.rotation(*ang)
    G = sphere.sh_grad_of_vectors(3, v)
    GR = sphere.sh_grad_of_vectors(3, v @ R.T)
    o = 0
    for l in range(4):
        D = sphere.wigner_d_real(l, *ang)
        blk = slice(o, o + 2 * l + 1)
        want = np.einsum("ab,ebk,jk->eaj", D, G[:, blk, :], R)
        assert np.allclose(GR[:, blk, :], want, atol=1e-12), l
        o += 2 * l + 1


def _axis_and_near_axis_vectors():
    # the +-z axis itself, points at sin(theta) = 1e-7 .. 0.49 from it (the rotation
    # branch), and points just past the switch-over at sin(theta) = 0.5
    v = [[0.0, 0.0, 1.0], [0.0, 0.0, -3.0], [0.0, 0.0, 0.25]]
    rng = np.random.default_rng(6)
    for s in (1e-7, 1e-4, 1e-2, 0.2, 0.49, 0.5, 0.51, 0.9):
        for sign in (1.0, -1.0):
            phi = rng.uniform(0, 2 * math.pi)
            r = rng.uniform(0.3, 3.0)
            v.append([r * s * math.cos(phi), r * s * math.sin(phi), sign * r * math.sqrt(1 - s * s)])
    return np.array(v)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_gradient_on_and_near_the_z_axis_matches_five_point_differences(L):
    # Y is smooth on the axis; only the polar-angle chain rule is singular there.  The
    # differences need no derivative formula, so they pin the rotation branch.
    v = _axis_and_near_axis_vectors()
    G = sphere.sh_grad_of_vectors(L, v)
    assert np.isfinite(G).all()
    r = np.linalg.norm(v, axis=1, keepdims=True)
    h = 1e-3 * r
    for k in range(3):
        d = np.zeros((1, 3))
        d[0, k] = 1.0
        f = [sphere.sh_of_vectors(L, v + t * h * d) for t in (-2, -1, 1, 2)]
        fd = (f[0] - 8 * f[1] + 8 * f[2] - f[3]) / (12 * h)
        assert np.abs((fd - G[:, :, k]) * r).max() < 1e-9, k


def test_gradient_on_the_z_axis_degree_one_closed_form():
    # sqrt(3) (e_k - n_k n) / r, the degree-1 closed form, at n = +-z exactly
    for n, r in (((0.0, 0.0, 1.0), 2.0), ((0.0, 0.0, -1.0), 0.5)):
        v = np.array([n]) * r
        G = sphere.sh_grad_of_vectors(1, v)[0]
        nn = np.array(n)
        for row, k in zip((1, 2, 3), (1, 2, 0)):
            e = np.zeros(3)
            e[k] = 1.0
            assert np.allclose(G[row], math.sqrt(3.0) * (e - nn[k] * nn) / r, atol=1e-14)


def test_gradient_branches_agree_where_both_are_regular():
    # between sin(theta) = 0.2 and 0.9 both the polar form and the rotation identity are
    # regular: they must give the same gradient
    rng = np.random.default_rng(7)
    s = rng.uniform(0.2, 0.9, 40)
    phi = rng.uniform(0, 2 * math.pi, 40)
    z = np.sqrt(1 - s * s) * np.where(rng.random(40) < 0.5, -1.0, 1.0)
    v = np.stack([s * np.cos(phi), s * np.sin(phi), z], axis=1) * rng.uniform(0.5, 2.0, (40, 1))
    R = sphere.rotation(0.0, math.pi / 2, 0.0)
    polar = sphere._sh_grad_polar(3, v)
    GR = sphere._sh_grad_polar(3, v @ R.T)
    o = 0
    for l in range(4):
        D = sphere.wigner_d_real(l, 0.0, math.pi / 2, 0.0)
        blk = slice(o, o + 2 * l + 1)
        rot = np.einsum("ba,ebk,kj->eaj", D, GR[:, blk, :], R)
        assert np.allclose(rot, polar[:, blk, :], atol=1e-12), l
        o += 2 * l + 1
