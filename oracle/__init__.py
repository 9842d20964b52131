"""CPU oracle for the fused UVU Clebsch-Gordan tensor-product convolution.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports, links or
calls anything here, and this package never touches the GPU library.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, see its header); this
module loads it with ctypes, converts arrays to fp64 and exposes:

  cg_complex, real_basis, cg_real_raw, cg_real, enumerate_paths   (tables)
  Desc                                                            (problem)
  fwd, bwd_edges, bwd_gx, dbwd, sender_csr                        (convolution)

and, in ``oracle.sphere``, test-only real spherical harmonics and real Wigner-D
matrices written from their textbook closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

BUILD_CMD = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", _SO, _SRC, "-lm"]


def build() -> str:
    """Compile liboracle.so next to its source (gcc, no GPU involvement)."""
    subprocess.run(BUILD_CMD, check=True)
    return _SO


_lib = None


def lib():
    """The oracle library.  ORACLE_SO names another build of oracle.c (the
    mutation tests load deliberately broken copies this way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_SO", _SO)
        if path == _SO and not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(path)
        d, i, i64, p = ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.oracle_cg_complex.restype = d
        L.oracle_cg_complex.argtypes = [i] * 6
        L.oracle_real_basis.restype = None
        L.oracle_real_basis.argtypes = [i, p, p]
        L.oracle_cg_real_raw.restype = i
        L.oracle_cg_real_raw.argtypes = [i, i, i, p, p]
        L.oracle_cg_real.restype = i
        L.oracle_cg_real.argtypes = [i, i, i, p]
        L.oracle_enumerate_paths.restype = i
        L.oracle_enumerate_paths.argtypes = [i, p, p, i, i, p, i]
        L.oracle_enumerate_paths_y.restype = i
        L.oracle_enumerate_paths_y.argtypes = [i, p, p, i, p, p, i, p, i]
        L.oracle_sender_csr.restype = None
        L.oracle_sender_csr.argtypes = [i64, i64, p, p, p]
        L.oracle_fwd.restype = i
        L.oracle_fwd.argtypes = [p, i64, i64, p, p, p, p, p, p, i64, p]
        L.oracle_bwd_edges.restype = i
        L.oracle_bwd_edges.argtypes = [p, i64, i64, p, p, p, p, p, p, p, i64, p, p]
        L.oracle_bwd_gx.restype = i
        L.oracle_bwd_gx.argtypes = [p, i64, i64, p, p, p, p, p, p, i64, p]
        L.oracle_dbwd.restype = i
        L.oracle_dbwd.argtypes = [p, i64, i64, p, p, p, p, p, p, p, p, p,
                                  p, i64, p, i64, p, i64, p, p, p, p]
        L.oracle_num_threads.restype = i
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [i]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _i64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int64)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(n)


# ---------------------------------------------------------------------------
# Tables
# ---------------------------------------------------------------------------

def cg_complex(j1, m1, j2, m2, J, M) -> float:
    return lib().oracle_cg_complex(j1, m1, j2, m2, J, M)


def real_basis(l: int) -> np.ndarray:
    n = 2 * l + 1
    re, im = np.zeros((n, n)), np.zeros((n, n))
    lib().oracle_real_basis(l, _ptr(re), _ptr(im))
    return re + 1j * im


def cg_real_raw(l1, l2, l3) -> np.ndarray:
    n1, n2, n3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
    re, im = np.zeros((n1, n2, n3)), np.zeros((n1, n2, n3))
    rc = lib().oracle_cg_real_raw(l1, l2, l3, _ptr(re), _ptr(im))
    if rc != 0:
        raise ValueError("l out of range")
    return re + 1j * im


def cg_real(l1, l2, l3) -> np.ndarray:
    n1, n2, n3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
    C = np.zeros((n1, n2, n3))
    rc = lib().oracle_cg_real(l1, l2, l3, _ptr(C))
    if rc < 0:
        raise ValueError("l out of range")
    return C


def enumerate_paths(x_irreps, y_lmax: int, l3_max: int, y_irreps=None):
    """[(i1, j, l3, p3), ...] for x irreps ((mul, l, parity), ...): j is the Y
    block, which for the default Y (degrees 0..y_lmax with parity (-1)^l) is the
    degree l2 itself."""
    xl = _i32([l for _, l, _ in x_irreps])
    xp = _i32([p for _, _, p in x_irreps])
    cap = 256
    out = np.zeros(4 * cap, dtype=np.int32)
    if y_irreps is None:
        n = lib().oracle_enumerate_paths(len(xl), _ptr(xl), _ptr(xp), y_lmax, l3_max,
                                         _ptr(out), cap)
    else:
        yl = _i32([l for _, l, _ in y_irreps])
        yp = _i32([p for _, _, p in y_irreps])
        n = lib().oracle_enumerate_paths_y(len(xl), _ptr(xl), _ptr(xp), len(yl), _ptr(yl),
                                           _ptr(yp), l3_max, _ptr(out), cap)
    assert n <= cap
    return [tuple(int(v) for v in out[4 * k:4 * k + 4]) for k in range(n)]


# ---------------------------------------------------------------------------
# Problem description
# ---------------------------------------------------------------------------

class _CDesc(ctypes.Structure):
    _fields_ = [("nx", ctypes.c_int), ("xl", ctypes.c_void_p), ("U", ctypes.c_int),
                ("ny", ctypes.c_int), ("yl", ctypes.c_void_p),
                ("np", ctypes.c_int), ("p_i1", ctypes.c_void_p),
                ("p_iy", ctypes.c_void_p), ("p_l3", ctypes.c_void_p),
                ("p_ob", ctypes.c_void_p), ("nob", ctypes.c_int),
                ("ob_l", ctypes.c_void_p), ("xm", ctypes.c_void_p), ("om", ctypes.c_void_p)]


class Desc:
    """x irreps (multiplicity U, or 1 for a block broadcast against the U channels),
    Y blocks, a path list and the output blocks (multiplicity U, or 1 for a block
    that sums the channels: out_mul).  Y: y_irreps ((1, l, parity), ...) in row order, or by default the
    harmonics of degrees 0..y_lmax with parity (-1)^l.  Paths are
    (x block, Y block, l3, output block); with the default Y the Y block index is
    the degree.  Default paths: all triangle-allowed ones up to l3_max, one output
    block per path, in enumeration order; or, given out_irreps ((mul, l, parity), ...),
    every enumerated path whose (l3, parity) is one of them, adding into that block."""

    def __init__(self, x_irreps, y_lmax: int, l3_max: int = 3,
                 paths: Optional[Sequence] = None, out_l: Optional[Sequence[int]] = None,
                 y_irreps=None, out_mul: Optional[Sequence[int]] = None, out_irreps=None):
        self.x_irreps = tuple(tuple(t) for t in x_irreps)
        self.U = max(m for m, _, _ in self.x_irreps)
        if any(m not in (1, self.U) for m, _, _ in self.x_irreps):
            raise ValueError("x blocks have U channels or one (broadcast)")
        if y_irreps is None:
            y_irreps = tuple((1, l, 1 if l % 2 == 0 else -1) for l in range(y_lmax + 1))
        self.y_irreps = tuple(tuple(t) for t in y_irreps)
        if any(m != 1 for m, _, _ in self.y_irreps):
            raise ValueError("Y blocks carry one channel each")
        self.yl = [l for _, l, _ in self.y_irreps]
        self.yoff = [int(v) for v in np.cumsum([0] + [2 * l + 1 for l in self.yl])[:-1]]
        self.L = max(self.yl)
        if paths is None and out_irreps is not None:
            outs = [(l, par) for _, l, par in out_irreps]
            en = enumerate_paths(self.x_irreps, y_lmax, l3_max, y_irreps=self.y_irreps)
            paths = [(i1, j, l3, outs.index((l3, p3))) for (i1, j, l3, p3) in en if (l3, p3) in outs]
            out_l = [l for l, _ in outs]
            out_mul = [m for m, _, _ in out_irreps]
        elif paths is None:
            en = enumerate_paths(self.x_irreps, y_lmax, l3_max, y_irreps=self.y_irreps)
            paths = [(i1, j, l3, k) for k, (i1, j, l3, _) in enumerate(en)]
            out_l = [l3 for (_, _, l3, _) in en]
        self.paths = [tuple(p) for p in paths]
        self.out_l = list(out_l)
        self.out_mul = [self.U] * len(self.out_l) if out_mul is None else list(out_mul)
        if len(self.out_mul) != len(self.out_l) or any(m not in (1, self.U) for m in self.out_mul):
            raise ValueError("output blocks have U channels or one (a sum over channels)")
        self.xl = [l for _, l, _ in self.x_irreps]
        self.xm = [m for m, _, _ in self.x_irreps]
        self.P = len(self.paths)
        self.x_dim = sum(m * (2 * l + 1) for m, l, _ in self.x_irreps)
        self.y_dim = sum(2 * l + 1 for l in self.yl)
        self.out_dim = sum(m * (2 * l + 1) for m, l in zip(self.out_mul, self.out_l))
        # keep the arrays alive for the C struct
        self._xl = _i32(self.xl)
        self._yl = _i32(self.yl)
        self._i1 = _i32([p[0] for p in self.paths])
        self._iy = _i32([p[1] for p in self.paths])
        self._l3 = _i32([p[2] for p in self.paths])
        self._ob = _i32([p[3] for p in self.paths])
        self._obl = _i32(self.out_l)
        self._xm = _i32(self.xm)
        self._om = _i32(self.out_mul)
        self._c = _CDesc(len(self.xl), _ptr(self._xl), self.U, len(self.yl), _ptr(self._yl), self.P,
                         _ptr(self._i1), _ptr(self._iy), _ptr(self._l3), _ptr(self._ob),
                         len(self.out_l), _ptr(self._obl), _ptr(self._xm), _ptr(self._om))

    def path_l2(self, p: int) -> int:
        """Degree of path p's Y block."""
        return self.yl[self.paths[p][1]]

    @property
    def cptr(self):
        return ctypes.byref(self._c)


# ---------------------------------------------------------------------------
# Convolution
# ---------------------------------------------------------------------------

def sender_csr(n_nodes: int, src: np.ndarray):
    src = _i32(src)
    srowptr = np.zeros(n_nodes + 1, dtype=np.int32)
    sperm = np.zeros(len(src), dtype=np.int32)
    lib().oracle_sender_csr(n_nodes, len(src), _ptr(src), _ptr(srowptr), _ptr(sperm))
    return srowptr, sperm


def _graph(rowptr, src):
    rowptr, src = _i32(rowptr), _i32(src)
    return rowptr, src, len(rowptr) - 1, len(src)


def fwd(d: Desc, rowptr, src, x, Y, W, rows=None) -> np.ndarray:
    rowptr, src, N, E = _graph(rowptr, src)
    x, Y, W, rows = _f64(x), _f64(Y), _f64(W), _i64(rows)
    nr = N if rows is None else len(rows)
    out = np.zeros((nr, d.out_dim))
    rc = lib().oracle_fwd(d.cptr, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W),
                          _ptr(rows), nr, _ptr(out))
    if rc != 0:
        raise ValueError("invalid description")
    return out


def bwd_edges(d: Desc, rowptr, src, x, Y, W, g, edges=None, want_gW=True, want_gY=True):
    rowptr, src, N, E = _graph(rowptr, src)
    x, Y, W, g, edges = _f64(x), _f64(Y), _f64(W), _f64(g), _i64(edges)
    ne = E if edges is None else len(edges)
    gW = np.zeros((ne, d.P, d.U)) if want_gW else None
    gY = np.zeros((ne, d.y_dim)) if want_gY else None
    rc = lib().oracle_bwd_edges(d.cptr, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y),
                                _ptr(W), _ptr(g), _ptr(edges), ne, _ptr(gW), _ptr(gY))
    if rc != 0:
        raise ValueError("invalid description")
    return gW, gY


def bwd_gx(d: Desc, rowptr, src, Y, W, g, senders=None) -> np.ndarray:
    rowptr, src, N, E = _graph(rowptr, src)
    Y, W, g, senders = _f64(Y), _f64(W), _f64(g), _i64(senders)
    ns = N if senders is None else len(senders)
    gx = np.zeros((ns, d.x_dim))
    rc = lib().oracle_bwd_gx(d.cptr, N, E, _ptr(rowptr), _ptr(src), _ptr(Y), _ptr(W),
                             _ptr(g), _ptr(senders), ns, _ptr(gx))
    if rc != 0:
        raise ValueError("invalid description")
    return gx


def bwd(d: Desc, rowptr, src, x, Y, W, g):
    """Full VJP: (gx, gY, gW)."""
    gW, gY = bwd_edges(d, rowptr, src, x, Y, W, g)
    gx = bwd_gx(d, rowptr, src, Y, W, g)
    return gx, gY, gW


def dbwd(d: Desc, rowptr, src, x, Y, W, g, ggx=None, ggY=None, ggW=None,
         rows=None, edges=None, senders=None, want=("dx", "dY", "dW", "dg")):
    """Double backward: dict with dx, dY, dW, dg (over the listed rows)."""
    rowptr, src, N, E = _graph(rowptr, src)
    x, Y, W, g = _f64(x), _f64(Y), _f64(W), _f64(g)
    ggx, ggY, ggW = _f64(ggx), _f64(ggY), _f64(ggW)
    rows, edges, senders = _i64(rows), _i64(edges), _i64(senders)
    nr = N if rows is None else len(rows)
    ne = E if edges is None else len(edges)
    ns = N if senders is None else len(senders)
    res = {
        "dx": np.zeros((ns, d.x_dim)) if "dx" in want else None,
        "dY": np.zeros((ne, d.y_dim)) if "dY" in want else None,
        "dW": np.zeros((ne, d.P, d.U)) if "dW" in want else None,
        "dg": np.zeros((nr, d.out_dim)) if "dg" in want else None,
    }
    rc = lib().oracle_dbwd(d.cptr, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W),
                           _ptr(g), _ptr(ggx), _ptr(ggY), _ptr(ggW), _ptr(rows), nr,
                           _ptr(edges), ne, _ptr(senders), ns, _ptr(res["dx"]),
                           _ptr(res["dY"]), _ptr(res["dW"]), _ptr(res["dg"]))
    if rc != 0:
        raise ValueError("invalid description")
    return res
