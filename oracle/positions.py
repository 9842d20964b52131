"""Test-only oracle of the convolution driven by atom positions (part of the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The receiver-major edge list comes from a neighbour list built on atom positions
("Receiver-streaming convolutions for channel-wise UVU tensor products", opening
post: the central atom is the receiver).  Reading: the vector of edge e = (s -> r)
is the neighbour's position relative to the central atom,
    vec[e] = pos[s] - pos[r],
and Y[e] holds the real spherical harmonics of its direction (oracle.sphere).  The
loss L = <g, f(x, Y(vec(pos)), W)> then depends on the positions through every
edge, and by the chain rule
    grad_vec[e] = sum_m grad_Y[e, m] dY[e, m] / dvec[e]
    grad_pos[n] = sum_{e: src[e] = n} grad_vec[e] - sum_{e in row n} grad_vec[e].
Each step is the plain definition: the oracle's VJP for grad_Y, the oracle's
harmonic gradient for dY/dvec, and a scatter-add (numpy.add.at) for the sums.
"""
from __future__ import annotations

import numpy as np

from . import bwd, fwd
from .sphere import sh_grad_of_vectors, sh_of_vectors


def receivers(rowptr) -> np.ndarray:
    rowptr = np.asarray(rowptr)
    return np.repeat(np.arange(len(rowptr) - 1), np.diff(rowptr))


def edge_vectors(rowptr, src, pos) -> np.ndarray:
    """vec[e] = pos[src[e]] - pos[receiver of e], [E, 3] in fp64."""
    pos = np.asarray(pos, dtype=np.float64)
    return pos[np.asarray(src)] - pos[receivers(rowptr)]


def _y_cols(d) -> np.ndarray:
    return np.concatenate([np.arange(l * l, (l + 1) ** 2) for l in d.yl])


def y_of_positions(d, rowptr, src, pos) -> np.ndarray:
    """The Y row of every edge for the descriptor's Y blocks (each the harmonics of its
    degree), from the positions."""
    return sh_of_vectors(max(d.yl), edge_vectors(rowptr, src, pos))[:, _y_cols(d)]


def fwd_pos(d, rowptr, src, x, pos, W) -> np.ndarray:
    return fwd(d, rowptr, src, x, y_of_positions(d, rowptr, src, pos), W)


def bwd_pos(d, rowptr, src, x, pos, W, g):
    """(grad_x, grad_pos, grad_W) of <g, f(x, Y(vec(pos)), W)>."""
    vec = edge_vectors(rowptr, src, pos)
    Y = sh_of_vectors(max(d.yl), vec)[:, _y_cols(d)]
    gx, gY, gW = bwd(d, rowptr, src, x, Y, W, g)
    gvec = np.einsum("em,emk->ek", gY, sh_grad_of_vectors(max(d.yl), vec)[:, _y_cols(d), :])
    gpos = np.zeros((len(rowptr) - 1, 3))
    np.add.at(gpos, np.asarray(src), gvec)
    np.add.at(gpos, receivers(rowptr), -gvec)
    return gx, gpos, gW
