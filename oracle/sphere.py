"""Test-only spherical harmonics and Wigner-D matrices (part of the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both are written from their textbook closed forms and carried to the real basis
with the oracle's change-of-basis matrix A_l (``oracle.real_basis``):

  * complex SH with the Condon-Shortley phase,
        Y_l^m = (-1)^m sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!) P_l^m(cos t) e^{i m p},  m >= 0,
        Y_l^{-m} = (-1)^m conj(Y_l^m),
    P_l^m the associated Legendre function without the phase, obtained by
    differentiating the Legendre polynomial m times; real, component-normalised
    SH are sqrt(4 pi) A_l Y_l.
  * Wigner's small-d formula and D^l_{m'm}(a,b,c) = e^{-i m' a} d^l_{m'm}(b) e^{-i m c}
    for the rotation R = Rz(a) Ry(b) Rz(c); the real matrix acting on real SH
    is A_l conj(D^l) A_l^H, the variant for which Y(R n) = D(R) Y(n).
"""
from __future__ import annotations

import math

import numpy as np
from numpy.polynomial import legendre as _leg
from numpy.polynomial import polynomial as _poly

from . import real_basis


def assoc_legendre(l: int, m: int, t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """P_l^m(t) = (1 - t^2)^(m/2) d^m P_l/dt^m (no Condon-Shortley phase), with
    s = sqrt(1 - t^2) = sin(theta) passed in (taken from the vector's components,
    which keeps it accurate near the z axis)."""
    c = np.zeros(l + 1)
    c[l] = 1.0
    p = _leg.leg2poly(c)
    dp = _poly.polyder(p, m) if m > 0 else p
    return s ** m * _poly.polyval(t, dp)


def sh_complex(l: int, vec: np.ndarray) -> np.ndarray:
    """Complex harmonics of unit vectors: cos(theta) = z, sin(theta) = sqrt(x^2 + y^2)."""
    x, y, z = vec[:, 0], vec[:, 1], vec[:, 2]
    t = np.clip(z, -1.0, 1.0)
    s = np.hypot(x, y)
    phi = np.arctan2(y, x)
    out = np.zeros((len(vec), 2 * l + 1), dtype=complex)
    for m in range(0, l + 1):
        n = math.sqrt((2 * l + 1) / (4 * math.pi) * math.factorial(l - m) / math.factorial(l + m))
        v = n * (-1) ** m * assoc_legendre(l, m, t, s) * np.exp(1j * m * phi)
        out[:, m + l] = v
        if m > 0:
            out[:, -m + l] = (-1) ** m * np.conj(v)
    return out


def sh_real(L: int, vec: np.ndarray) -> np.ndarray:
    """[E, (L+1)^2] real component-normalised SH, degrees 0..L, m = -l..l."""
    cols = []
    for l in range(L + 1):
        yl = math.sqrt(4 * math.pi) * (sh_complex(l, vec) @ real_basis(l).T)
        assert np.abs(yl.imag).max(initial=0.0) < 1e-12
        cols.append(yl.real)
    return np.concatenate(cols, axis=1)


def sh_of_vectors(L: int, vec: np.ndarray) -> np.ndarray:
    """Real component-normalised SH of the directions of vectors of any length,
    [E, (L+1)^2].  A zero vector has no direction: it gets Y_00 = 1 and zeros."""
    vec = np.asarray(vec, dtype=np.float64)
    r = np.linalg.norm(vec, axis=1)
    live = r > 0
    n = np.zeros_like(vec)
    n[live] = vec[live] / r[live, None]
    n[~live] = (0.0, 0.0, 1.0)
    Y = sh_real(L, n)
    Y[~live, 1:] = 0.0
    return Y


def _legendre_parts(l: int, m: int):
    """q = d^m P_l / dt^m and q' as polynomial coefficient arrays."""
    c = np.zeros(l + 1)
    c[l] = 1.0
    q = _poly.polyder(_leg.leg2poly(c), m) if m > 0 else _leg.leg2poly(c)
    return q, _poly.polyder(q)


def _sh_grad_polar(L: int, vec: np.ndarray) -> np.ndarray:
    """Gradient of sh_of_vectors with respect to the vector, [E, (L+1)^2, 3], by
    the chain rule through the polar angles:
        grad Y = (dY/dtheta) e_theta / r + (dY/dphi) e_phi / (r sin theta),
    dY/dphi = i m Y for the complex harmonics, and for P_l^m(t) = (1-t^2)^(m/2) q(t),
    t = cos theta: dP/dtheta = -sin(theta)^(m-1) [sin^2(theta) q'(t) - m cos(theta) q(t)]
    (m = 0: -sin(theta) q'(t)); then carried to the real basis like the values.
    Undefined on the z axis (sin theta = 0) for m > 0; zero for a zero vector."""
    vec = np.asarray(vec, dtype=np.float64)
    E = len(vec)
    r = np.linalg.norm(vec, axis=1)
    live = r > 0
    x, y, z = (vec[:, k] / np.where(live, r, 1.0) for k in range(3))
    ct = np.clip(z, -1.0, 1.0)
    st = np.hypot(x, y)
    phi = np.arctan2(y, x)
    e_theta = np.stack([ct * np.cos(phi), ct * np.sin(phi), -st], axis=1)
    e_phi = np.stack([-np.sin(phi), np.cos(phi), np.zeros(E)], axis=1)
    rr = np.where(live, r, 1.0)
    cols = []
    for l in range(L + 1):
        gc = np.zeros((E, 2 * l + 1, 3), dtype=complex)
        for m in range(0, l + 1):
            nrm = math.sqrt((2 * l + 1) / (4 * math.pi) * math.factorial(l - m) / math.factorial(l + m))
            q, dq = _legendre_parts(l, m)
            qv, dqv = _poly.polyval(ct, q), _poly.polyval(ct, dq)
            if m == 0:
                dP = -st * dqv
                P_over_s = np.zeros(E)          # multiplied by m = 0 below
            else:
                dP = -st ** (m - 1) * (st * st * dqv - m * ct * qv)
                P_over_s = st ** (m - 1) * qv   # P_l^m / sin(theta)
            ph = np.exp(1j * m * phi)
            dtheta = nrm * (-1) ** m * dP * ph
            dphi_over_s = nrm * (-1) ** m * P_over_s * ph * (1j * m)
            g = (dtheta[:, None] * e_theta + dphi_over_s[:, None] * e_phi) / rr[:, None]
            gc[:, m + l, :] = g
            if m > 0:
                gc[:, -m + l, :] = (-1) ** m * np.conj(g)
        A = real_basis(l)
        gl = math.sqrt(4 * math.pi) * np.einsum("mk,ekd->emd", A, gc)
        assert np.abs(gl.imag).max(initial=0.0) < 1e-9
        cols.append(gl.real)
    G = np.concatenate(cols, axis=1)
    G[~live] = 0.0
    return G


# Rotation used to carry vectors off the z axis: R = Ry(pi/2) takes the z axis to the x axis.
_OFF_AXIS = (0.0, math.pi / 2, 0.0)


def sh_grad_of_vectors(L: int, vec: np.ndarray) -> np.ndarray:
    """Gradient of sh_of_vectors with respect to the vector, [E, (L+1)^2, 3],
    defined for every vector.

    Away from the z axis it is the polar-angle chain rule (_sh_grad_polar).  Within
    sin(theta) < 0.5 of the axis it comes from the rotation identity instead: the
    harmonics satisfy Y(R v) = D(R) Y(v), so Y(v) = D(R)^T Y(R v) and
        grad Y(v) = D(R)^T grad Y(R v) R,
    with R = Ry(pi/2), which takes every such vector to sin(theta) > 0.85, where
    the polar form is regular.  D is the real Wigner-D of this module.  Zero for a
    zero vector."""
    vec = np.asarray(vec, dtype=np.float64)
    G = _sh_grad_polar(L, vec)
    r = np.linalg.norm(vec, axis=1)
    live = r > 0
    sin_t = np.zeros(len(vec))
    sin_t[live] = np.hypot(vec[live, 0], vec[live, 1]) / r[live]
    near = live & (sin_t < 0.5)
    if near.any():
        R = rotation(*_OFF_AXIS)
        GR = _sh_grad_polar(L, vec[near] @ R.T)
        o = 0
        for l in range(L + 1):
            D = wigner_d_real(l, *_OFF_AXIS)
            blk = slice(o, o + 2 * l + 1)
            G[near, blk, :] = np.einsum("ba,ebk,kj->eaj", D, GR[:, blk, :], R)
            o += 2 * l + 1
    return G


def small_d(l: int, mp: int, m: int, beta: float) -> float:
    s = 0.0
    cb, sb = math.cos(beta / 2), math.sin(beta / 2)
    for k in range(0, 2 * l + 1):
        a = (l + m - k, k, l - k - mp, k - m + mp)
        if min(a) < 0:
            continue
        num = math.sqrt(math.factorial(l + mp) * math.factorial(l - mp) *
                        math.factorial(l + m) * math.factorial(l - m))
        den = (math.factorial(a[0]) * math.factorial(a[1]) * math.factorial(a[2]) *
               math.factorial(a[3]))
        s += (-1) ** (k - m + mp) * num / den * cb ** (2 * l - 2 * k + m - mp) * \
            sb ** (2 * k - m + mp)
    return s


def wigner_d_complex(l: int, a: float, b: float, c: float) -> np.ndarray:
    D = np.zeros((2 * l + 1, 2 * l + 1), dtype=complex)
    for mp in range(-l, l + 1):
        for m in range(-l, l + 1):
            D[mp + l, m + l] = np.exp(-1j * mp * a) * small_d(l, mp, m, b) * np.exp(-1j * m * c)
    return D


def wigner_d_real(l: int, a: float, b: float, c: float) -> np.ndarray:
    A = real_basis(l)
    D = A @ wigner_d_complex(l, a, b, c).conj() @ A.conj().T
    assert np.abs(D.imag).max() < 1e-12
    return D.real


def rot_z(t: float) -> np.ndarray:
    c, s = math.cos(t), math.sin(t)
    return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])


def rot_y(t: float) -> np.ndarray:
    c, s = math.cos(t), math.sin(t)
    return np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]])


def rotation(a: float, b: float, c: float) -> np.ndarray:
    return rot_z(a) @ rot_y(b) @ rot_z(c)


def block_diag_irreps(blocks, a, b, c):
    """Real Wigner-D acting on a feature row laid out as blocks [(U, l), ...],
    each block u-major (element u*(2l+1)+m)."""
    mats = []
    for U, l in blocks:
        D = wigner_d_real(l, a, b, c)
        mats.append(np.kron(np.eye(U), D))
    n = sum(m.shape[0] for m in mats)
    out = np.zeros((n, n))
    o = 0
    for m in mats:
        k = m.shape[0]
        out[o:o + k, o:o + k] = m
        o += k
    return out
