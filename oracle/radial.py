"""Radial weights from edge lengths: the oracle (part of the test infrastructure,
like the rest of this package; see its docstring).

The pages leave the radial weights outside the kernels: they are realised
beforehand, and fusing their realisation would be a new operation
("Receiver-streaming convolutions for channel-wise UVU tensor products",
maintainer replies).  They give no specification, so this one is a plain,
stated reading (the form used by MACE-style potentials):

  r = |vec|, d = r / r_cut
  envelope  u(d) = 1 - (p+1)(p+2)/2 d^p + p(p+2) d^(p+1) - p(p+1)/2 d^(p+2)  for d < 1, else 0;  p = 6
  basis     B_n(r) = sqrt(2 / r_cut) sin(n pi r / r_cut) / r * u(d),  n = 1..NB,  NB = 8
            (at r = 0 the limit sqrt(2 / r_cut) n pi / r_cut)
  hidden    pre = B W1 / sqrt(NB),  h = silu(pre) = pre * sigmoid(pre)       W1: [NB, H]
  weights   W = h W2 / sqrt(H)                                               W2: [H, P*U]

Plain fp64 numpy, written out step by step; the backward is the chain rule of
the same steps, in the same order.
"""
from __future__ import annotations

import math

import numpy as np

NB = 8
P_ENV = 6


def envelope(d: np.ndarray) -> np.ndarray:
    p = P_ENV
    d = np.asarray(d, dtype=np.float64)
    u = (1.0 - (p + 1) * (p + 2) / 2.0 * d ** p + p * (p + 2) * d ** (p + 1)
         - p * (p + 1) / 2.0 * d ** (p + 2))
    return np.where(d < 1.0, u, 0.0)


def envelope_deriv(d: np.ndarray) -> np.ndarray:
    """du/dd = -p(p+1)(p+2)/2 d^(p-1) (1 - d)^2 for d < 1, else 0."""
    p = P_ENV
    d = np.asarray(d, dtype=np.float64)
    return np.where(d < 1.0, -p * (p + 1) * (p + 2) / 2.0 * d ** (p - 1) * (1.0 - d) ** 2, 0.0)


def bessel_basis(r: np.ndarray, r_cut: float) -> np.ndarray:
    """[E, NB] radial basis of lengths r."""
    r = np.asarray(r, dtype=np.float64)
    n = np.arange(1, NB + 1, dtype=np.float64)
    k = n * math.pi / r_cut
    c = math.sqrt(2.0 / r_cut)
    safe = np.where(r > 0, r, 1.0)
    s = np.where(r[:, None] > 0, np.sin(k[None, :] * r[:, None]) / safe[:, None], k[None, :])
    return c * s * envelope(r / r_cut)[:, None]


def bessel_basis_deriv(r: np.ndarray, r_cut: float) -> np.ndarray:
    """[E, NB] dB_n/dr (0 at r = 0, where the basis is even in r)."""
    r = np.asarray(r, dtype=np.float64)
    n = np.arange(1, NB + 1, dtype=np.float64)
    k = n * math.pi / r_cut
    c = math.sqrt(2.0 / r_cut)
    safe = np.where(r > 0, r, 1.0)[:, None]
    kr = k[None, :] * r[:, None]
    s = np.sin(kr) / safe                                   # sin(kr)/r
    ds = (k[None, :] * np.cos(kr) * safe - np.sin(kr)) / safe ** 2
    d = r / r_cut
    out = c * (ds * envelope(d)[:, None] + s * envelope_deriv(d)[:, None] / r_cut)
    return np.where(r[:, None] > 0, out, 0.0)


def silu(x):
    return x / (1.0 + np.exp(-x))


def silu_deriv(x):
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def radial_fwd(vec, r_cut: float, W1, W2):
    """W [E, P*U] from edge vectors vec [E, 3]."""
    vec = np.asarray(vec, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    H = W1.shape[1]
    r = np.linalg.norm(vec, axis=1)
    B = bessel_basis(r, r_cut)
    pre = B @ W1 / math.sqrt(NB)
    h = silu(pre)
    return h @ W2 / math.sqrt(H)


def radial_bwd(vec, r_cut: float, W1, W2, gW):
    """Gradients of <gW, radial_fwd(vec, r_cut, W1, W2)> with respect to vec,
    W1 and W2."""
    vec = np.asarray(vec, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    gW = np.asarray(gW, dtype=np.float64)
    H = W1.shape[1]
    r = np.linalg.norm(vec, axis=1)
    B = bessel_basis(r, r_cut)
    pre = B @ W1 / math.sqrt(NB)
    h = silu(pre)
    dh = gW @ W2.T / math.sqrt(H)
    gW2 = h.T @ gW / math.sqrt(H)
    dpre = dh * silu_deriv(pre)
    gW1 = B.T @ dpre / math.sqrt(NB)
    dB = dpre @ W1.T / math.sqrt(NB)
    dr = np.sum(dB * bessel_basis_deriv(r, r_cut), axis=1)
    safe = np.where(r > 0, r, 1.0)
    gvec = np.where(r[:, None] > 0, dr[:, None] * vec / safe[:, None], 0.0)
    return gvec, gW1, gW2
