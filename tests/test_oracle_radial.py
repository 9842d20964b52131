"""Pins of the radial-weight oracle (oracle/radial.py): the envelope's boundary
values and smoothness, the orthonormality of the sine basis, the r -> 0 limit,
and the backward against five-point finite differences of the forward along
random directions of every argument."""
import math

import numpy as np
import pytest

from oracle import radial

RC = 6.0


def test_envelope_boundary_and_smoothness():
    assert radial.envelope(np.array([0.0]))[0] == 1.0
    assert abs(radial.envelope(np.array([1.0 - 1e-12]))[0]) < 1e-12
    assert radial.envelope(np.array([1.0, 1.5]))[0] == 0.0
    # first and second derivatives vanish at the cutoff (second by differences of the first)
    assert abs(radial.envelope_deriv(np.array([1.0 - 1e-9]))[0]) < 1e-12
    # u'' ~ p(p+1)(p+2)(1 - d) near the cutoff: the difference quotient shrinks with the step
    for h, bound in ((1e-4, 0.06), (1e-6, 6e-4)):
        d2 = (radial.envelope_deriv(np.array([1.0 - h]))[0] - radial.envelope_deriv(np.array([1.0 - 2 * h]))[0]) / h
        assert abs(d2) < bound
    d = np.linspace(0.0, 1.0, 201)
    assert np.all(np.diff(radial.envelope(d)) <= 1e-15)             # decreasing
    # derivative against five-point differences
    x = np.linspace(0.05, 0.95, 19)
    hh = 1e-4
    fd = (radial.envelope(x - 2 * hh) - 8 * radial.envelope(x - hh) + 8 * radial.envelope(x + hh)
          - radial.envelope(x + 2 * hh)) / (12 * hh)
    assert np.allclose(fd, radial.envelope_deriv(x), atol=1e-9)


def test_sine_basis_orthonormal_on_the_cutoff_interval():
    # r B_n(r) / u(r/r_c) = sqrt(2/r_c) sin(n pi r / r_c): orthonormal on [0, r_c]
    r = (np.arange(20000) + 0.5) * RC / 20000                        # midpoint rule
    B = radial.bessel_basis(r, RC) * r[:, None] / radial.envelope(r / RC)[:, None]
    G = B.T @ B * (RC / 20000)
    assert np.allclose(G, np.eye(radial.NB), atol=1e-7)


def test_basis_limit_at_zero_and_cutoff():
    n = np.arange(1, radial.NB + 1)
    B0 = radial.bessel_basis(np.array([0.0]), RC)[0]
    assert np.allclose(B0, math.sqrt(2 / RC) * n * math.pi / RC, atol=0)
    Bs = radial.bessel_basis(np.array([1e-7]), RC)[0]
    assert np.allclose(Bs, B0, rtol=1e-9)
    assert not radial.bessel_basis(np.array([RC, RC + 1.0]), RC).any()
    r = np.linspace(0.3, 5.9, 50)
    hh = 1e-5
    fd = (radial.bessel_basis(r - 2 * hh, RC) - 8 * radial.bessel_basis(r - hh, RC)
          + 8 * radial.bessel_basis(r + hh, RC) - radial.bessel_basis(r + 2 * hh, RC)) / (12 * hh)
    assert np.allclose(fd, radial.bessel_basis_deriv(r, RC), atol=1e-8)


def _problem(seed, E=40, H=16, PU=24):
    rng = np.random.default_rng(seed)
    vec = rng.standard_normal((E, 3))
    vec *= (rng.uniform(0.5, 5.5, E) / np.linalg.norm(vec, axis=1))[:, None]
    return vec, rng.standard_normal((radial.NB, H)), rng.standard_normal((H, PU)), rng.standard_normal((E, PU))


def test_silu_derivative():
    x = np.linspace(-6, 6, 41)
    h = 1e-4
    fd = (radial.silu(x - 2 * h) - 8 * radial.silu(x - h) + 8 * radial.silu(x + h) - radial.silu(x + 2 * h)) / (12 * h)
    assert np.allclose(fd, radial.silu_deriv(x), atol=1e-10)


@pytest.mark.parametrize("which", ["vec", "W1", "W2"])
def test_backward_against_differences(which):
    vec, W1, W2, gW = _problem(3)
    gvec, gW1, gW2 = radial.radial_bwd(vec, RC, W1, W2, gW)
    rng = np.random.default_rng(9)
    args = {"vec": vec, "W1": W1, "W2": W2}
    grad = {"vec": gvec, "W1": gW1, "W2": gW2}[which]
    d = rng.standard_normal(args[which].shape)
    h = 1e-4

    def f(t):
        a = dict(args)
        a[which] = args[which] + t * d
        return np.sum(gW * radial.radial_fwd(a["vec"], RC, a["W1"], a["W2"]))
    fd = (f(-2 * h) - 8 * f(-h) + 8 * f(h) - f(2 * h)) / (12 * h)
    assert abs(fd - np.sum(grad * d)) <= 1e-8 * max(1.0, abs(fd))


def test_linear_in_W2():
    vec, W1, W2, _ = _problem(4)
    a = radial.radial_fwd(vec, RC, W1, W2)
    b = radial.radial_fwd(vec, RC, W1, 2.0 * W2 - 1.0)
    c = radial.radial_fwd(vec, RC, W1, np.ones_like(W2))
    assert np.allclose(b, 2.0 * a - c, atol=1e-12)
