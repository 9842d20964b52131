"""Pins of the oracle's gradient to atom positions (oracle/positions.py), against
what the mathematics fixes: five-point finite differences of the loss in every
position coordinate, translation invariance (the gradients sum to zero; the loss
does not change), rotation equivariance through the real Wigner-D, and zero
contribution from self-loops (a zero edge vector has no direction)."""
import math

import numpy as np
import pytest

import oracle
from oracle import positions, sphere

DESCS = [
    dict(x_irreps=((3, 0, 1), (3, 1, -1)), y_lmax=2, l3_max=2),
    dict(x_irreps=((2, 0, 1), (2, 1, -1), (2, 2, 1)), y_lmax=3, l3_max=3),
    dict(x_irreps=((2, 1, -1), (2, 2, 1)), y_lmax=0, l3_max=3, y_irreps=((1, 3, -1), (1, 1, -1))),
]


def _problem(k, seed, self_loops=False):
    rng = np.random.default_rng(seed)
    d = oracle.Desc(**DESCS[k])
    N = 7
    deg = rng.integers(1, 5, size=N)
    rowptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    E = int(rowptr[-1])
    recv = np.repeat(np.arange(N), deg)
    src = rng.integers(0, N - 1, size=E)
    src = (src + (src >= recv)).astype(np.int32)          # no self-loops
    if self_loops:
        src[0] = recv[0]
        src[-1] = recv[-1]
    pos = rng.uniform(-2.0, 2.0, size=(N, 3))
    x = rng.standard_normal((N, d.x_dim))
    W = rng.standard_normal((E, d.P, d.U))
    g = rng.standard_normal((N, d.out_dim))
    return d, rowptr, src, pos, x, W, g


def _loss(d, rowptr, src, x, pos, W, g):
    return float(np.vdot(g, positions.fwd_pos(d, rowptr, src, x, pos, W)))


@pytest.mark.parametrize("k", range(len(DESCS)))
def test_grad_pos_matches_five_point_differences(k):
    d, rowptr, src, pos, x, W, g = _problem(k, 50 + k)
    _, gpos, _ = positions.bwd_pos(d, rowptr, src, x, pos, W, g)
    h = 1e-3
    fd = np.zeros_like(pos)
    for n in range(len(pos)):
        for c in range(3):
            vals = []
            for t in (-2, -1, 1, 2):
                p = pos.copy()
                p[n, c] += t * h
                vals.append(_loss(d, rowptr, src, x, p, W, g))
            fd[n, c] = (vals[0] - 8 * vals[1] + 8 * vals[2] - vals[3]) / (12 * h)
    assert np.abs(fd - gpos).max() <= 1e-8 * max(1.0, np.abs(gpos).max())


@pytest.mark.parametrize("k", range(len(DESCS)))
def test_translation_invariance(k):
    d, rowptr, src, pos, x, W, g = _problem(k, 60 + k)
    gx, gpos, gW = positions.bwd_pos(d, rowptr, src, x, pos, W, g)
    assert np.abs(gpos.sum(axis=0)).max() <= 1e-12 * np.abs(gpos).max()
    t = np.array([0.3, -1.7, 2.2])
    assert math.isclose(_loss(d, rowptr, src, x, pos + t, W, g), _loss(d, rowptr, src, x, pos, W, g),
                        rel_tol=1e-12, abs_tol=1e-12)
    gx2, gpos2, gW2 = positions.bwd_pos(d, rowptr, src, x, pos + t, W, g)
    assert np.allclose(gpos2, gpos, atol=1e-12) and np.allclose(gx2, gx, atol=1e-12)


@pytest.mark.parametrize("k", [0, 1])
def test_rotation_equivariance_of_grad_pos(k):
    """L(R pos, D x, W, D g) = L(pos, x, W, g), so grad_pos(R pos, D x, W, D g) = R grad_pos(pos, x, W, g)."""
    d, rowptr, src, pos, x, W, g = _problem(k, 70 + k)
    ang = (0.4, 1.3, -0.8)
    R = sphere.rotation(*ang)
    Dx = sphere.block_diag_irreps([(d.U, l) for l in d.xl], *ang)
    Do = sphere.block_diag_irreps([(d.U, l) for l in d.out_l], *ang)
    _, gpos, _ = positions.bwd_pos(d, rowptr, src, x, pos, W, g)
    _, gposR, _ = positions.bwd_pos(d, rowptr, src, x @ Dx.T, pos @ R.T, W, g @ Do.T)
    assert np.allclose(gposR, gpos @ R.T, atol=1e-11)


def test_self_loops_contribute_nothing_to_grad_pos():
    d, rowptr, src, pos, x, W, g = _problem(1, 80, self_loops=True)
    _, gpos, _ = positions.bwd_pos(d, rowptr, src, x, pos, W, g)
    keep = np.ones(len(src), dtype=bool)
    recv = positions.receivers(rowptr)
    keep[src == recv] = False
    assert (~keep).sum() == 2
    # dropping the self-loops (and their weights) changes grad_pos only through f's other
    # outputs, not at all: a zero vector has no direction and a zero harmonic gradient
    rp = np.concatenate([[0], np.cumsum(np.bincount(recv[keep], minlength=len(pos)))]).astype(np.int32)
    _, gpos_k, _ = positions.bwd_pos(d, rp, src[keep], x, pos, W[keep], g)
    assert np.allclose(gpos, gpos_k, atol=1e-12)
