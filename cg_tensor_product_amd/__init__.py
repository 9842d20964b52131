"""Python binding of liboeq.so, the MI355X library for the fused channel-wise
(UVU) Clebsch-Gordan tensor-product graph convolution.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch provides device memory and the current HIP stream.  The
binding allocates outputs (and the deterministic-mode workspace) with torch and
passes raw pointers; the library itself never allocates in a compute call.

Names follow the C ABI (include/oeq.h):
  Plan (oeq_plan_create / oeq_plan_dims / oeq_plan_paths / oeq_plan_destroy)
  oeq_tp_conv_fwd, oeq_tp_conv_bwd, oeq_tp_conv_dbwd, oeq_workspace_size,
  oeq_cg_table, oeq_sender_csr, oeq_csr_check.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboeq.so")

OEQ_F32, OEQ_F64 = 0, 1
OEQ_BWD_ATOMIC, OEQ_BWD_DETERMINISTIC = 0, 1
_MODES = {"atomic": OEQ_BWD_ATOMIC, "deterministic": OEQ_BWD_DETERMINISTIC}
STATUS = {0: "OEQ_OK", 1: "OEQ_ERR_INVALID_ARG", 2: "OEQ_ERR_UNSUPPORTED", 3: "OEQ_ERR_WORKSPACE",
          4: "OEQ_ERR_HIP", 5: "OEQ_ERR_JIT"}

EXPORTED = ["oeq_plan_create", "oeq_plan_create_cached", "oeq_plan_destroy", "oeq_plan_dims", "oeq_plan_paths", "oeq_plan_code_key",
            "oeq_cg_table",
            "oeq_workspace_size", "oeq_tp_conv_fwd", "oeq_tp_conv_bwd", "oeq_tp_conv_bwd_noalloc", "oeq_tp_conv_dbwd",
            "oeq_csr_workspace_size", "oeq_sender_csr", "oeq_csr_check", "oeq_status_string",
            "oeq_last_error", "oeq_plan_schedule", "oeq_sender_view", "oeq_tp_conv_fwd_sender",
            "oeq_tp_conv_bwd_sender", "oeq_sph_harm", "oeq_sph_harm_bwd", "oeq_tp_conv_fwd_vec",
            "oeq_workspace_size_vec", "oeq_tp_conv_bwd_vec", "oeq_radial_workspace_size", "oeq_radial_fwd",
            "oeq_radial_bwd", "oeq_tp_conv_fwd_radial", "oeq_workspace_size_radial", "oeq_tp_conv_bwd_radial",
            "oeq_tp_conv_fwd_pos", "oeq_workspace_size_pos", "oeq_tp_conv_bwd_pos"]
SCHEDULES = {0: "receiver", 1: "sender"}


class OeqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class _Irrep(ctypes.Structure):
    _fields_ = [("mul", ctypes.c_int32), ("l", ctypes.c_int32), ("parity", ctypes.c_int32)]


class _Path(ctypes.Structure):
    _fields_ = [("in1", ctypes.c_int32), ("in2", ctypes.c_int32), ("out", ctypes.c_int32)]


class _Desc(ctypes.Structure):
    _fields_ = [("x_irreps", ctypes.POINTER(_Irrep)), ("n_x", ctypes.c_int32),
                ("y_irreps", ctypes.POINTER(_Irrep)), ("n_y", ctypes.c_int32),
                ("y_lmax", ctypes.c_int32), ("out_irreps", ctypes.POINTER(_Irrep)),
                ("n_out", ctypes.c_int32), ("paths", ctypes.POINTER(_Path)),
                ("n_paths", ctypes.c_int32), ("lmax_out", ctypes.c_int32), ("dtype", ctypes.c_int)]


_lib = None


def lib():
    """The loaded liboeq.so.  Raises if the library has not been built: there is
    no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int
    L.oeq_plan_create.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(P)]
    L.oeq_plan_create.restype = st
    L.oeq_plan_create_cached.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(P)]
    L.oeq_plan_create_cached.restype = st
    L.oeq_plan_destroy.argtypes = [P]
    L.oeq_plan_destroy.restype = None
    L.oeq_plan_dims.argtypes = [P] + [ctypes.POINTER(I64)] * 5
    L.oeq_plan_dims.restype = st
    L.oeq_plan_paths.argtypes = [P, P, I32]
    L.oeq_plan_paths.restype = st
    L.oeq_plan_code_key.argtypes = [P, ctypes.c_char_p, SZ]
    L.oeq_plan_code_key.restype = st
    L.oeq_cg_table.argtypes = [I32, I32, I32, P]
    L.oeq_cg_table.restype = st
    L.oeq_workspace_size.argtypes = [P, I64, I64, ctypes.c_int, ctypes.POINTER(SZ)]
    L.oeq_workspace_size.restype = st
    L.oeq_tp_conv_fwd.argtypes = [P, I64, I64, P, P, P, P, P, P, P]
    L.oeq_tp_conv_fwd.restype = st
    L.oeq_tp_conv_bwd.argtypes = [P, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int, P, SZ, P]
    L.oeq_tp_conv_bwd.restype = st
    L.oeq_tp_conv_bwd_noalloc.argtypes = [P, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int, P]
    L.oeq_tp_conv_bwd_noalloc.restype = st
    L.oeq_tp_conv_dbwd.argtypes = [P, I64, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int, P, SZ, P]
    L.oeq_tp_conv_dbwd.restype = st
    L.oeq_csr_workspace_size.argtypes = [I64, I64, ctypes.POINTER(SZ)]
    L.oeq_csr_workspace_size.restype = st
    L.oeq_sender_csr.argtypes = [I64, I64, P, P, P, P, SZ, P]
    L.oeq_sender_csr.restype = st
    L.oeq_csr_check.argtypes = [I64, I64, P, P, P]
    L.oeq_csr_check.restype = st
    L.oeq_plan_schedule.argtypes = [P, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    L.oeq_plan_schedule.restype = st
    L.oeq_sender_view.argtypes = [I64, I64, P, P, P, P, P, P, SZ, P]
    L.oeq_sender_view.restype = st
    L.oeq_tp_conv_fwd_sender.argtypes = [P, I64, I64, P, P, P, P, P, P, P, P]
    L.oeq_tp_conv_fwd_sender.restype = st
    L.oeq_tp_conv_bwd_sender.argtypes = [P, I64, I64, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.oeq_tp_conv_bwd_sender.restype = st
    L.oeq_sph_harm.argtypes = [P, I64, P, P, P]
    L.oeq_sph_harm.restype = st
    L.oeq_sph_harm_bwd.argtypes = [P, I64, P, P, P, P]
    L.oeq_sph_harm_bwd.restype = st
    L.oeq_tp_conv_fwd_vec.argtypes = [P, I64, I64, P, P, P, P, P, P, P]
    L.oeq_tp_conv_fwd_vec.restype = st
    L.oeq_workspace_size_vec.argtypes = [P, I64, I64, ctypes.c_int, ctypes.POINTER(SZ)]
    L.oeq_workspace_size_vec.restype = st
    L.oeq_tp_conv_bwd_vec.argtypes = [P, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int, P, SZ, P]
    L.oeq_tp_conv_bwd_vec.restype = st
    L.oeq_tp_conv_fwd_pos.argtypes = [P, I64, I64, P, P, P, P, P, P, P]
    L.oeq_tp_conv_fwd_pos.restype = st
    L.oeq_workspace_size_pos.argtypes = [P, I64, I64, ctypes.c_int, ctypes.POINTER(SZ)]
    L.oeq_workspace_size_pos.restype = st
    L.oeq_tp_conv_bwd_pos.argtypes = [P, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int, P, SZ, P]
    L.oeq_tp_conv_bwd_pos.restype = st
    D = ctypes.c_double
    L.oeq_radial_workspace_size.argtypes = [P, I64, I32, ctypes.POINTER(SZ)]
    L.oeq_radial_workspace_size.restype = st
    L.oeq_radial_fwd.argtypes = [P, I64, P, D, I32, P, P, P, P, SZ, P]
    L.oeq_radial_fwd.restype = st
    L.oeq_radial_bwd.argtypes = [P, I64, P, D, I32, P, P, P, P, P, P, P, SZ, P]
    L.oeq_radial_bwd.restype = st
    L.oeq_tp_conv_fwd_radial.argtypes = [P, I64, I64, P, P, P, P, P, D, P, P, P, P, SZ, P]
    L.oeq_tp_conv_fwd_radial.restype = st
    L.oeq_workspace_size_radial.argtypes = [P, I64, I64, ctypes.c_int, ctypes.POINTER(SZ)]
    L.oeq_workspace_size_radial.restype = st
    L.oeq_tp_conv_bwd_radial.argtypes = [P, I64, I64, P, P, P, P, P, D, P, P, P, P, P, P, P, P, ctypes.c_int, P, SZ,
                                         P]
    L.oeq_tp_conv_bwd_radial.restype = st
    L.oeq_status_string.argtypes = [ctypes.c_int]
    L.oeq_status_string.restype = ctypes.c_char_p
    L.oeq_last_error.argtypes = []
    L.oeq_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise OeqError(status, lib().oeq_last_error().decode())


def _irreps(seq) -> tuple:
    if isinstance(seq, str):
        out = []
        for part in seq.split("+"):
            mul, rest = part.strip().split("x")
            out.append((int(mul), int(rest[:-1]), 1 if rest[-1] == "e" else -1))
        return tuple(out)
    return tuple(tuple(int(v) for v in t) for t in seq)


class Plan:
    """oeq_plan_create for an irreps descriptor.  dtype: "f32" or "f64".

    x and output blocks have U channels (the largest x multiplicity) or one: a
    one-channel x block is broadcast against the U channels, a one-channel output
    block (out_irreps) receives their sum.

    Y: y_irreps (one-channel irreps in row order, e.g. "1x0e+1x2e+1x1e"), or by
    default the spherical harmonics of degrees 0..y_lmax.  paths=None enumerates
    every triangle-allowed path up to lmax_out; an explicit list holds
    (x block, Y block, output block) triples and needs out_irreps (with the default
    Y the Y block index is the degree)."""

    def __init__(self, x_irreps, y_lmax: int, lmax_out: int = 3, dtype: str = "f32",
                 paths: Optional[Sequence] = None, out_irreps=None, y_irreps=None):
        self.x_irreps = _irreps(x_irreps)
        self.y_irreps = None if y_irreps is None else _irreps(y_irreps)
        self.y_lmax = int(y_lmax)
        self.lmax_out = int(lmax_out)
        self.dtype = dtype
        xs = (_Irrep * len(self.x_irreps))(*[_Irrep(*t) for t in self.x_irreps])
        d = _Desc()
        d.x_irreps = xs
        d.n_x = len(self.x_irreps)
        d.y_lmax = self.y_lmax
        d.lmax_out = self.lmax_out
        d.dtype = OEQ_F64 if dtype == "f64" else OEQ_F32
        if dtype not in ("f32", "f64"):
            d.dtype = 7  # rejected by the library
        keep = [xs]
        if self.y_irreps is not None:
            ys = (_Irrep * len(self.y_irreps))(*[_Irrep(*t) for t in self.y_irreps])
            d.y_irreps, d.n_y = ys, len(self.y_irreps)
            keep.append(ys)
        if out_irreps is not None:
            oi = _irreps(out_irreps)
            os_ = (_Irrep * len(oi))(*[_Irrep(*t) for t in oi])
            d.out_irreps, d.n_out = os_, len(oi)
            keep.append(os_)
        if paths is not None:
            ps = (_Path * len(paths))(*[_Path(*t) for t in paths])
            d.paths, d.n_paths = ps, len(paths)
            keep.append(ps)
        h = ctypes.c_void_p()
        # the library compiles a plan missing from its code-object cache in its compiler
        # helper (a child process), so the kernels do not depend on what this process loaded
        st = lib().oeq_plan_create(ctypes.byref(d), ctypes.byref(h))
        _check(st)
        self._h = h
        dims = [ctypes.c_int64() for _ in range(5)]
        _check(lib().oeq_plan_dims(h, *[ctypes.byref(v) for v in dims]))
        self.x_dim, self.y_dim, self.out_dim, self.n_paths, self.w_per_edge = (int(v.value) for v in dims)
        self.U = self.w_per_edge // self.n_paths  # channels: the largest x multiplicity

    @property
    def handle(self):
        return self._h

    def paths(self):
        """[(x block, l1, l2, l3, output block, output parity), ...]"""
        buf = np.zeros(6 * self.n_paths, dtype=np.int32)
        _check(lib().oeq_plan_paths(self._h, buf.ctypes.data, self.n_paths))
        return [tuple(int(v) for v in buf[6 * k:6 * k + 6]) for k in range(self.n_paths)]

    @property
    def code_key(self) -> str:
        """Hash identifying the compiled kernels of this plan."""
        buf = ctypes.create_string_buffer(64)
        _check(lib().oeq_plan_code_key(self._h, buf, 64))
        return buf.value.decode()

    def schedule(self):
        """oeq_plan_schedule: {"fwd": "receiver"|"sender", "bwd": ..., "move_fwd": [r, s],
        "move_bwd": [r, s]} (the data-movement model's per-edge, per-channel elements)."""
        f, b = ctypes.c_int(), ctypes.c_int()
        mf, mb = (ctypes.c_double * 2)(), (ctypes.c_double * 2)()
        _check(lib().oeq_plan_schedule(self._h, ctypes.byref(f), ctypes.byref(b), mf, mb))
        return {"fwd": SCHEDULES[f.value], "bwd": SCHEDULES[b.value], "move_fwd": list(mf), "move_bwd": list(mb)}

    def torch_dtype(self):
        import torch
        return torch.float64 if self.dtype == "f64" else torch.float32

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.oeq_plan_destroy(h)
            self._h = None


def oeq_cg_table(l1: int, l2: int, l3: int) -> np.ndarray:
    out = np.zeros((2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1))
    _check(lib().oeq_cg_table(l1, l2, l3, out.ctypes.data))
    return out.reshape(2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)


def oeq_workspace_size(plan: Plan, n_nodes: int, n_edges: int, mode: str = "atomic") -> int:
    b = ctypes.c_size_t()
    _check(lib().oeq_workspace_size(plan.handle, n_nodes, n_edges, _MODES[mode], ctypes.byref(b)))
    return int(b.value)


# ---------------------------------------------------------------------------
# tensor helpers
# ---------------------------------------------------------------------------

def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _want(t, shape, dtype, name):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _graph(rowptr, src):
    import torch
    N = rowptr.shape[0] - 1
    E = src.shape[0]
    _want(rowptr, (N + 1,), torch.int32, "rowptr")
    _want(src, (E,), torch.int32, "src")
    return N, E


def _empty(shape, dtype, device):
    import torch
    return torch.empty(shape, dtype=dtype, device=device)


def _workspace(plan, N, E, mode, device):
    import torch
    nbytes = oeq_workspace_size(plan, N, E, mode)
    if nbytes == 0:
        return None, 0
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes], nbytes


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def oeq_tp_conv_fwd(plan: Plan, rowptr, src, x, Y, W, out=None):
    """out[N, out_dim] = f(x, Y, W) (receiver-stationary forward)."""
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(Y, (E, plan.y_dim), dt, "Y")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    if out is None:
        out = _empty((N, plan.out_dim), dt, rowptr.device)
    _want(out, (N, plan.out_dim), dt, "out")
    _check(lib().oeq_tp_conv_fwd(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W),
                                 _ptr(out), _stream()))
    return out


def oeq_tp_conv_bwd(plan: Plan, rowptr, src, x, Y, W, grad_out, mode: str = "atomic",
                    need=("x", "Y", "W"), out=None, workspace=None):
    """(grad_x, grad_Y, grad_W) of <grad_out, f(x, Y, W)>; entries not in `need`
    are None.  `out` may supply preallocated (grad_x, grad_Y, grad_W)."""
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(Y, (E, plan.y_dim), dt, "Y")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    _want(grad_out, (N, plan.out_dim), dt, "grad_out")
    dev = rowptr.device
    shapes = ((N, plan.x_dim), (E, plan.y_dim), (E, plan.n_paths, plan.U))
    if out is None:
        out = tuple(_empty(s, dt, dev) if k in need else None for k, s in zip(("x", "Y", "W"), shapes))
    gx, gY, gW = (_want(t, s, dt, n) for t, s, n in zip(out, shapes, ("grad_x", "grad_Y", "grad_W")))
    ws, nbytes = (workspace, workspace.numel()) if workspace is not None else _workspace(plan, N, E, mode, dev)
    _check(lib().oeq_tp_conv_bwd(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W),
                                 _ptr(grad_out), _ptr(gx), _ptr(gY), _ptr(gW), _MODES[mode], _ptr(ws), nbytes,
                                 _stream()))
    return gx, gY, gW


def oeq_tp_conv_bwd_noalloc(plan: Plan, rowptr, src, x, Y, W, grad_out, out, mode: str = "atomic"):
    """oeq_tp_conv_bwd into preallocated (grad_x, grad_Y, grad_W) (None: not computed),
    with the library's fixed device scratch in place of a workspace."""
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(Y, (E, plan.y_dim), dt, "Y")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    _want(grad_out, (N, plan.out_dim), dt, "grad_out")
    shapes = ((N, plan.x_dim), (E, plan.y_dim), (E, plan.n_paths, plan.U))
    gx, gY, gW = (_want(t, s, dt, n) for t, s, n in zip(out, shapes, ("grad_x", "grad_Y", "grad_W")))
    _check(lib().oeq_tp_conv_bwd_noalloc(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W),
                                         _ptr(grad_out), _ptr(gx), _ptr(gY), _ptr(gW), _MODES[mode], _stream()))
    return gx, gY, gW


def oeq_tp_conv_dbwd(plan: Plan, rowptr, src, x, Y, W, grad_out, gg_x=None, gg_Y=None, gg_W=None,
                     mode: str = "atomic", want=("x", "Y", "W", "grad_out"), workspace=None, out=None):
    """Double backward: dict with d_x, d_Y, d_W, d_grad_out (None if not in want).
    out: optional dict of preallocated outputs with the same keys (a missing or None
    entry is not requested); it overrides want."""
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(Y, (E, plan.y_dim), dt, "Y")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    _want(grad_out, (N, plan.out_dim), dt, "grad_out")
    _want(gg_x, (N, plan.x_dim), dt, "gg_x")
    _want(gg_Y, (E, plan.y_dim), dt, "gg_Y")
    _want(gg_W, (E, plan.n_paths, plan.U), dt, "gg_W")
    dev = rowptr.device
    shapes = {"x": (N, plan.x_dim), "Y": (E, plan.y_dim), "W": (E, plan.n_paths, plan.U),
              "grad_out": (N, plan.out_dim)}
    if out is not None:
        d = {k: out.get(k) for k in shapes}
        for k, t in d.items():
            _want(t, shapes[k], dt, "d_" + k)
    else:
        d = {k: _empty(shp, dt, dev) if k in want else None for k, shp in shapes.items()}
    ws, nbytes = (workspace, workspace.numel()) if workspace is not None else _workspace(plan, N, E, mode, dev)
    _check(lib().oeq_tp_conv_dbwd(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(W),
                                  _ptr(grad_out), _ptr(gg_x), _ptr(gg_Y), _ptr(gg_W), _ptr(d["x"]), _ptr(d["Y"]),
                                  _ptr(d["W"]), _ptr(d["grad_out"]), _MODES[mode], _ptr(ws), nbytes, _stream()))
    return d


def oeq_sender_csr(src, n_nodes: int):
    """Device sender CSR: (srowptr[N+1], sperm[E]) int32."""
    import torch
    E = src.shape[0]
    _want(src, (E,), torch.int32, "src")
    b = ctypes.c_size_t()
    _check(lib().oeq_csr_workspace_size(n_nodes, E, ctypes.byref(b)))
    ws = torch.empty(int(b.value) + 256, dtype=torch.uint8, device=src.device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + int(b.value)]
    srowptr = torch.empty(n_nodes + 1, dtype=torch.int32, device=src.device)
    sperm = torch.empty(E, dtype=torch.int32, device=src.device)
    _check(lib().oeq_sender_csr(n_nodes, E, _ptr(src), _ptr(srowptr), _ptr(sperm), _ptr(ws), int(b.value),
                                _stream()))
    return srowptr, sperm


def oeq_csr_check(rowptr, src) -> None:
    N, E = _graph(rowptr, src)
    _check(lib().oeq_csr_check(N, E, _ptr(rowptr), _ptr(src), _stream()))


def oeq_sender_view(rowptr, src):
    """Device sender view (srowptr[N+1], sperm[E], sdst[E]) int32 of a receiver CSR."""
    import torch
    N, E = _graph(rowptr, src)
    dev = src.device
    srowptr = torch.empty(N + 1, dtype=torch.int32, device=dev)
    sperm = torch.empty(max(E, 1), dtype=torch.int32, device=dev)[:E]
    sdst = torch.empty(max(E, 1), dtype=torch.int32, device=dev)[:E]
    nbytes = ctypes.c_size_t()
    _check(lib().oeq_csr_workspace_size(N, E, ctypes.byref(nbytes)))
    raw = torch.empty(nbytes.value + 256, dtype=torch.uint8, device=dev)
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + nbytes.value]
    _check(lib().oeq_sender_view(N, E, _ptr(rowptr), _ptr(src), _ptr(srowptr), _ptr(sperm), _ptr(sdst), _ptr(ws),
                                 nbytes.value, _stream()))
    return srowptr, sperm, sdst


def oeq_tp_conv_fwd_sender(plan: Plan, view, x, Y, W, out=None):
    """Sender-stationary forward; view = oeq_sender_view(rowptr, src)."""
    srowptr, sperm, sdst = view
    N, E = srowptr.shape[0] - 1, sperm.shape[0]
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(Y, (E, plan.y_dim), dt, "Y")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    if out is None:
        out = _empty((N, plan.out_dim), dt, x.device)
    _want(out, (N, plan.out_dim), dt, "out")
    _check(lib().oeq_tp_conv_fwd_sender(plan.handle, N, E, _ptr(srowptr), _ptr(sperm), _ptr(sdst), _ptr(x), _ptr(Y),
                                        _ptr(W), _ptr(out), _stream()))
    return out


def oeq_tp_conv_bwd_sender(plan: Plan, view, x, Y, W, grad_out, want=("x", "Y", "W"), out=None, workspace=None):
    """Sender-stationary VJP: (grad_x, grad_Y, grad_W), None where not in want."""
    srowptr, sperm, sdst = view
    N, E = srowptr.shape[0] - 1, sperm.shape[0]
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(Y, (E, plan.y_dim), dt, "Y")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    _want(grad_out, (N, plan.out_dim), dt, "grad_out")
    shapes = ((N, plan.x_dim), (E, plan.y_dim), (E, plan.n_paths, plan.U))
    if out is None:
        out = tuple(_empty(shp, dt, x.device) if k in want else None for k, shp in zip(("x", "Y", "W"), shapes))
    for t, shp, k in zip(out, shapes, ("grad_x", "grad_Y", "grad_W")):
        _want(t, shp, dt, k)
    ws, nbytes = (workspace, workspace.numel()) if workspace is not None else _workspace(plan, N, E, "atomic",
                                                                                        x.device)
    _check(lib().oeq_tp_conv_bwd_sender(plan.handle, N, E, _ptr(srowptr), _ptr(sperm), _ptr(sdst), _ptr(x), _ptr(Y),
                                        _ptr(W), _ptr(grad_out), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(ws),
                                        nbytes, _stream()))
    return out


def oeq_sph_harm(plan: Plan, vec, out=None):
    """Y[E, (L+1)^2] of edge vectors vec[E, 3]."""
    E = vec.shape[0]
    dt = plan.torch_dtype()
    _want(vec, (E, 3), dt, "vec")
    if out is None:
        out = _empty((E, plan.y_dim), dt, vec.device)
    _want(out, (E, plan.y_dim), dt, "Y")
    _check(lib().oeq_sph_harm(plan.handle, E, _ptr(vec), _ptr(out), _stream()))
    return out


def oeq_sph_harm_bwd(plan: Plan, vec, grad_Y, out=None):
    """grad_vec[E, 3] = sum_m grad_Y[e, m] dY[e, m] / dvec[e]."""
    E = vec.shape[0]
    dt = plan.torch_dtype()
    _want(vec, (E, 3), dt, "vec")
    _want(grad_Y, (E, plan.y_dim), dt, "grad_Y")
    if out is None:
        out = _empty((E, 3), dt, vec.device)
    _want(out, (E, 3), dt, "grad_vec")
    _check(lib().oeq_sph_harm_bwd(plan.handle, E, _ptr(vec), _ptr(grad_Y), _ptr(out), _stream()))
    return out


def oeq_tp_conv_fwd_vec(plan: Plan, rowptr, src, x, vec, W, out=None):
    """Forward with Y evaluated in the kernel from the edge vectors."""
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(vec, (E, 3), dt, "vec")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    if out is None:
        out = _empty((N, plan.out_dim), dt, rowptr.device)
    _want(out, (N, plan.out_dim), dt, "out")
    _check(lib().oeq_tp_conv_fwd_vec(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(vec), _ptr(W),
                                     _ptr(out), _stream()))
    return out


def oeq_workspace_size_vec(plan: Plan, n_nodes: int, n_edges: int, mode: str = "atomic") -> int:
    b = ctypes.c_size_t()
    _check(lib().oeq_workspace_size_vec(plan.handle, n_nodes, n_edges, _MODES[mode], ctypes.byref(b)))
    return b.value


def oeq_tp_conv_bwd_vec(plan: Plan, rowptr, src, x, vec, W, grad_out, mode: str = "atomic",
                        want=("x", "vec", "W"), out=None, workspace=None):
    """VJP to (x, vec, W) of the forward from edge vectors."""
    import torch
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(vec, (E, 3), dt, "vec")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    _want(grad_out, (N, plan.out_dim), dt, "grad_out")
    shapes = ((N, plan.x_dim), (E, 3), (E, plan.n_paths, plan.U))
    if out is None:
        out = tuple(_empty(shp, dt, x.device) if k in want else None for k, shp in zip(("x", "vec", "W"), shapes))
    for t, shp, k in zip(out, shapes, ("grad_x", "grad_vec", "grad_W")):
        _want(t, shp, dt, k)
    if workspace is None:
        nbytes = oeq_workspace_size_vec(plan, N, E, mode)
        raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=x.device)
        workspace = raw[(-raw.data_ptr()) % 256:][:nbytes]
    _check(lib().oeq_tp_conv_bwd_vec(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(vec), _ptr(W),
                                     _ptr(grad_out), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _MODES[mode],
                                     _ptr(workspace), workspace.numel(), _stream()))
    return out


def oeq_tp_conv_fwd_pos(plan: Plan, rowptr, src, x, pos, W, out=None):
    """Forward with Y evaluated in the kernel from atom positions pos[N, 3]
    (vec[e] = pos[src[e]] - pos[receiver])."""
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(pos, (N, 3), dt, "pos")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    if out is None:
        out = _empty((N, plan.out_dim), dt, rowptr.device)
    _want(out, (N, plan.out_dim), dt, "out")
    _check(lib().oeq_tp_conv_fwd_pos(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(pos), _ptr(W),
                                     _ptr(out), _stream()))
    return out


def oeq_workspace_size_pos(plan: Plan, n_nodes: int, n_edges: int, mode: str = "atomic") -> int:
    b = ctypes.c_size_t()
    _check(lib().oeq_workspace_size_pos(plan.handle, n_nodes, n_edges, _MODES[mode], ctypes.byref(b)))
    return b.value


def oeq_tp_conv_bwd_pos(plan: Plan, rowptr, src, x, pos, W, grad_out, mode: str = "atomic",
                        want=("x", "pos", "W"), out=None, workspace=None):
    """VJP to (x, pos, W) of the forward from atom positions."""
    import torch
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(pos, (N, 3), dt, "pos")
    _want(W, (E, plan.n_paths, plan.U), dt, "W")
    _want(grad_out, (N, plan.out_dim), dt, "grad_out")
    shapes = ((N, plan.x_dim), (N, 3), (E, plan.n_paths, plan.U))
    if out is None:
        out = tuple(_empty(shp, dt, x.device) if k in want else None for k, shp in zip(("x", "pos", "W"), shapes))
    for t, shp, k in zip(out, shapes, ("grad_x", "grad_pos", "grad_W")):
        _want(t, shp, dt, k)
    if workspace is None:
        nbytes = oeq_workspace_size_pos(plan, N, E, mode)
        raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=x.device)
        workspace = raw[(-raw.data_ptr()) % 256:][:nbytes]
    _check(lib().oeq_tp_conv_bwd_pos(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(pos), _ptr(W),
                                     _ptr(grad_out), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _MODES[mode],
                                     _ptr(workspace), workspace.numel(), _stream()))
    return out


def _radial_ws(plan, E, hidden, device):
    import torch
    b = ctypes.c_size_t()
    _check(lib().oeq_radial_workspace_size(plan.handle, E, hidden, ctypes.byref(b)))
    raw = torch.empty(b.value + 256, dtype=torch.uint8, device=device)
    return raw[(-raw.data_ptr()) % 256:][:b.value]


def oeq_radial_fwd(plan: Plan, vec, r_cut: float, W1, W2, out=None, workspace=None):
    """Radial weights W [E, P, U] from edge vectors (see oeq.h for the form)."""
    E = vec.shape[0]
    dt = plan.torch_dtype()
    H = W1.shape[1]
    _want(vec, (E, 3), dt, "vec")
    _want(W1, (8, H), dt, "W1")
    _want(W2, (H, plan.n_paths * plan.U), dt, "W2")
    if out is None:
        out = _empty((E, plan.n_paths, plan.U), dt, vec.device)
    _want(out, (E, plan.n_paths, plan.U), dt, "W")
    ws = workspace if workspace is not None else _radial_ws(plan, E, H, vec.device)
    _check(lib().oeq_radial_fwd(plan.handle, E, _ptr(vec), float(r_cut), H, _ptr(W1), _ptr(W2), _ptr(out), _ptr(ws),
                                ws.numel(), _stream()))
    return out


def oeq_radial_bwd(plan: Plan, vec, r_cut: float, W1, W2, grad_W, want=("vec", "W1", "W2"), workspace=None):
    """(grad_vec, grad_W1, grad_W2) of <grad_W, W(vec, W1, W2)>; None where not in want."""
    E = vec.shape[0]
    dt = plan.torch_dtype()
    H = W1.shape[1]
    _want(vec, (E, 3), dt, "vec")
    _want(W1, (8, H), dt, "W1")
    _want(W2, (H, plan.n_paths * plan.U), dt, "W2")
    _want(grad_W, (E, plan.n_paths, plan.U), dt, "grad_W")
    gv = _empty((E, 3), dt, vec.device) if "vec" in want else None
    g1 = _empty((8, H), dt, vec.device) if "W1" in want else None
    g2 = _empty((H, plan.n_paths * plan.U), dt, vec.device) if "W2" in want else None
    ws = workspace if workspace is not None else _radial_ws(plan, E, H, vec.device)
    _check(lib().oeq_radial_bwd(plan.handle, E, _ptr(vec), float(r_cut), H, _ptr(W1), _ptr(W2), _ptr(grad_W),
                                _ptr(gv), _ptr(g1), _ptr(g2), _ptr(ws), ws.numel(), _stream()))
    return gv, g1, g2


def oeq_tp_conv_fwd_radial(plan: Plan, rowptr, src, x, Y, vec, r_cut: float, W1, W2, out=None, workspace=None):
    """Forward with W formed in the kernel from a hidden width of 8 (W1 [8, 8], W2 [8, P*U])."""
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(Y, (E, plan.y_dim), dt, "Y")
    _want(vec, (E, 3), dt, "vec")
    _want(W1, (8, 8), dt, "W1")
    _want(W2, (8, plan.n_paths * plan.U), dt, "W2")
    if out is None:
        out = _empty((N, plan.out_dim), dt, x.device)
    _want(out, (N, plan.out_dim), dt, "out")
    ws = workspace if workspace is not None else _radial_ws(plan, E, 8, x.device)
    _check(lib().oeq_tp_conv_fwd_radial(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(vec),
                                        float(r_cut), _ptr(W1), _ptr(W2), _ptr(out), _ptr(ws), ws.numel(),
                                        _stream()))
    return out


def oeq_tp_conv_bwd_radial(plan: Plan, rowptr, src, x, Y, vec, r_cut: float, W1, W2, grad_out, mode: str = "atomic",
                           want=("x", "Y", "vec", "W1", "W2"), workspace=None):
    """VJP of oeq_tp_conv_fwd_radial: dict with grad_x, grad_Y, grad_vec, grad_W1, grad_W2
    (None where not in want)."""
    import torch
    N, E = _graph(rowptr, src)
    dt = plan.torch_dtype()
    _want(x, (N, plan.x_dim), dt, "x")
    _want(Y, (E, plan.y_dim), dt, "Y")
    _want(vec, (E, 3), dt, "vec")
    _want(W1, (8, 8), dt, "W1")
    _want(W2, (8, plan.n_paths * plan.U), dt, "W2")
    _want(grad_out, (N, plan.out_dim), dt, "grad_out")
    shapes = {"x": (N, plan.x_dim), "Y": (E, plan.y_dim), "vec": (E, 3), "W1": (8, 8),
              "W2": (8, plan.n_paths * plan.U)}
    out = {k: _empty(shp, dt, x.device) if k in want else None for k, shp in shapes.items()}
    if workspace is None:
        b = ctypes.c_size_t()
        _check(lib().oeq_workspace_size_radial(plan.handle, N, E, _MODES[mode], ctypes.byref(b)))
        raw = torch.empty(b.value + 256, dtype=torch.uint8, device=x.device)
        workspace = raw[(-raw.data_ptr()) % 256:][:b.value]
    _check(lib().oeq_tp_conv_bwd_radial(plan.handle, N, E, _ptr(rowptr), _ptr(src), _ptr(x), _ptr(Y), _ptr(vec),
                                        float(r_cut), _ptr(W1), _ptr(W2), _ptr(grad_out), _ptr(out["x"]),
                                        _ptr(out["Y"]), _ptr(out["vec"]), _ptr(out["W1"]), _ptr(out["W2"]),
                                        _MODES[mode], _ptr(workspace), workspace.numel(), _stream()))
    return out
