"""Seeded synthetic inputs for the UVU CG tensor-product convolution.

This module is shared by the tests, the smoke check and the benchmark.  It
draws random numbers and lays them out; it contains none of the convolution's
arithmetic (no Clebsch-Gordan coefficients, no path rules, no contraction).

Workloads follow "Receiver-streaming convolutions for channel-wise UVU tensor
products" (opening post, benchmark paragraph): a synthetic receiver-sorted
graph of 5,000 nodes and 280,000 edges with a uniform in-degree of 56.  The
other sizes are the small cases used for parity tests.

Recipe (every tensor from its own child of one SeedSequence):
  * graph:  each receiver r draws its in-degree's worth of distinct senders
            uniformly from {0..N-1} minus {r}, sorted ascending inside the row;
            the edge id is the position in that receiver-major order.  Multigraph
            workloads (edge-case tests) draw with replacement from all N nodes
            instead: self-loops and repeated (s, r) edges.
  * edge vectors: z ~ N(0, I3), normalised; Y = real spherical harmonics of
            them with component normalisation (sum over m of Y^2 = 2l+1),
            degrees 0..L, m = -l..l, l=1 ordered (y, z, x); a workload with
            listed Y blocks gets the harmonics of each block's degree.
  * x, g, v ~ N(0,1); W ~ N(0,1) * w_scale.
  * values are drawn in fp64 and rounded to nearest-even for fp32 workloads,
    so the fp64 twin of a workload sees the same draws.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

# Child stream indices of the workload's SeedSequence.
_GRAPH, _VEC, _X, _W, _G, _V, _EXTRA = range(7)
_NCHILD = 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_nodes: int
    degree: int                      # uniform in-degree (ignored if degrees given)
    x_irreps: tuple                  # ((mul, l, parity), ...), parity +1 'e' / -1 'o'
    y_lmax: int
    l3_max: int
    dtype: str                       # "f32" | "f64"
    w_scale: str                     # "unit" | "inv_sqrt_paths"
    seed: int
    ops: tuple = ("fwd", "bwd")
    degrees: Optional[tuple] = None  # per-receiver in-degree (non-uniform graphs)
    multi: bool = False              # senders drawn with replacement, the receiver included
    y_irreps: Optional[tuple] = None # Y blocks ((1, l, parity), ...); None: degrees 0..y_lmax
    one_sender: bool = False         # every edge leaves node 0 (counter calibration: x is one row)
    out_irreps: Optional[tuple] = None  # output blocks ((mul, l, parity), ...), mul U or 1; None: one per path

    @property
    def U(self) -> int:
        return max(m for m, _, _ in self.x_irreps)

    @property
    def n_edges(self) -> int:
        if self.degrees is not None:
            return int(sum(self.degrees))
        return self.n_nodes * self.degree

    @property
    def x_dim(self) -> int:
        return sum(mul * (2 * l + 1) for mul, l, _ in self.x_irreps)

    @property
    def y_degrees(self) -> tuple:
        if self.y_irreps is None:
            return tuple(range(self.y_lmax + 1))
        return tuple(l for _, l, _ in self.y_irreps)

    @property
    def y_dim(self) -> int:
        return sum(2 * l + 1 for l in self.y_degrees)

    def np_dtype(self):
        return np.float64 if self.dtype == "f64" else np.float32

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _irr(s: str):
    """'128x0e+128x1o' -> ((128, 0, 1), (128, 1, -1))."""
    out = []
    for part in s.split("+"):
        mul, rest = part.split("x")
        out.append((int(mul), int(rest[:-1]), 1 if rest[-1] == "e" else -1))
    return tuple(out)


WORKLOADS = {
    # 64 nodes, in-degree 16, 8x0e+8x1o, Y l<=2, outputs l3<=1, fp64.
    "tiny_fp64": Workload("tiny_fp64", 64, 16, _irr("8x0e+8x1o"), 2, 1, "f64", "unit", 1001),
    # 5,000 nodes / 280,000 edges, 128x0e+128x1o, Y l<=3, l3<=3, fp32, W ~ N(0,1)/sqrt(P).
    "mace_medium_fp32": Workload("mace_medium_fp32", 5000, 56, _irr("128x0e+128x1o"), 3, 3,
                                 "f32", "inv_sqrt_paths", 2002),
    # Same graph and draws in fp64.
    "mace_medium_fp64": Workload("mace_medium_fp64", 5000, 56, _irr("128x0e+128x1o"), 3, 3,
                                 "f64", "inv_sqrt_paths", 2002),
    # 128x0e+128x1o+128x2e, fp32, forward + VJP + HVP.
    "mace_large_fp32": Workload("mace_large_fp32", 5000, 56, _irr("128x0e+128x1o+128x2e"), 3, 3,
                                "f32", "inv_sqrt_paths", 4004, ("fwd", "bwd", "hvp")),
    # 256x0e+256x1o+256x2e, fp32, W ~ N(0,1) materialised (multi-GB).
    "wide_proxy_fp32": Workload("wide_proxy_fp32", 5000, 56, _irr("256x0e+256x1o+256x2e"), 3, 3,
                                "f32", "unit", 5005, ("fwd", "bwd", "hvp")),
    # Invariant (l3 = 0) outputs of degree-0..3 features: 128x0e+128x1o+128x2e+128x3o, 4 paths.
    # An x row is four times wider than an output row: the shape for which moving
    # output rows (sender-stationary) is cheaper than moving x rows.
    "invariant_fp32": Workload("invariant_fp32", 5000, 56, _irr("128x0e+128x1o+128x2e+128x3o"), 3, 0,
                               "f32", "inv_sqrt_paths", 6006),
}


# UVW products that reduce to the channel-wise one, at the medium workload's sizes (same
# graph and seeds): a broadcast scalar beside 128 vector channels, and outputs of which the
# pseudotensor and scalar blocks sum the channels.
REDUCIBLE = {
    "uvw_bcast_medium_fp32": Workload("uvw_bcast_medium_fp32", 5000, 56, _irr("1x0e+128x1o"), 3, 3, "f32",
                                      "inv_sqrt_paths", 2002),
    "uvw_sum_medium_fp32": Workload("uvw_sum_medium_fp32", 5000, 56, _irr("128x0e+128x1o"), 3, 3, "f32",
                                    "inv_sqrt_paths", 2002,
                                    out_irreps=_irr("1x0e+128x1o+128x2e+128x3o+1x1e+1x2o+1x3e")),
}


# Counter calibration: the medium workload's sizes with every edge leaving node 0, so the
# forward's HBM reads are the non-temporal W stream, Y and the CSR (x is a single cached
# row); FETCH_SIZE of that forward checks the counter's scale for the kernels' own loads.
CALIBRATION = {
    "nt_read_calibration_fp32": Workload("nt_read_calibration_fp32", 5000, 56, _irr("128x0e+128x1o"), 3, 3,
                                         "f32", "inv_sqrt_paths", 2002, one_sender=True),
}


def by_name(name: str) -> Workload:
    """A workload of WORKLOADS, REDUCIBLE or CALIBRATION."""
    for table in (WORKLOADS, REDUCIBLE, CALIBRATION):
        if name in table:
            return table[name]
    raise KeyError(name)


# ---------------------------------------------------------------------------
# Graph
# ---------------------------------------------------------------------------

def make_graph(n_nodes: int, degrees: Sequence[int], rng: np.random.Generator, multi: bool = False):
    """Receiver-sorted CSR: rowptr[N+1] (int32), src[E] (int32).

    multi=False: distinct senders other than the receiver (a neighbour list).
    multi=True: senders drawn uniformly with replacement from all N nodes, so a row
    may hold self-loops (s = r) and repeated (s, r) edges; still sorted in the row."""
    degrees = np.asarray(degrees, dtype=np.int64)
    assert degrees.shape == (n_nodes,)
    if not multi and n_nodes > 0 and degrees.max(initial=0) > n_nodes - 1:
        raise ValueError("in-degree larger than N-1 cannot have distinct senders")
    rowptr = np.zeros(n_nodes + 1, dtype=np.int64)
    np.cumsum(degrees, out=rowptr[1:])
    E = int(rowptr[-1])
    if E >= 2**31:
        raise ValueError("edge count exceeds int32 CSR")
    src = np.empty(E, dtype=np.int32)
    for r in range(n_nodes):
        d = int(degrees[r])
        if d == 0:
            continue
        if multi:
            v = rng.integers(0, n_nodes, size=d)
        else:
            v = rng.choice(n_nodes - 1, size=d, replace=False)
            v = v + (v >= r)         # skip the receiver itself
        v.sort()
        src[rowptr[r]:rowptr[r + 1]] = v
    return rowptr.astype(np.int32), src


# ---------------------------------------------------------------------------
# Edge attributes: real spherical harmonics (Cartesian polynomials)
# ---------------------------------------------------------------------------

def real_sh_cartesian(L: int, vec: np.ndarray) -> np.ndarray:
    """Component-normalised real spherical harmonics of unit vectors, degrees 0..L
    (L <= 3), m = -l..l, from the Cartesian polynomial forms.  vec: [E, 3]."""
    x, y, z = vec[:, 0], vec[:, 1], vec[:, 2]
    cols = [np.ones_like(x)]
    if L >= 1:
        s3 = math.sqrt(3.0)
        cols += [s3 * y, s3 * z, s3 * x]
    if L >= 2:
        s15, s5 = math.sqrt(15.0), math.sqrt(5.0)
        cols += [s15 * x * y, s15 * y * z, 0.5 * s5 * (3 * z * z - 1.0),
                 s15 * x * z, 0.5 * s15 * (x * x - y * y)]
    if L >= 3:
        a, b, c = math.sqrt(35.0 / 8.0), math.sqrt(105.0), math.sqrt(21.0 / 8.0)
        cols += [a * y * (3 * x * x - y * y), b * x * y * z, c * y * (5 * z * z - 1.0),
                 0.5 * math.sqrt(7.0) * (5 * z ** 3 - 3 * z), c * x * (5 * z * z - 1.0),
                 0.5 * b * z * (x * x - y * y), a * x * (x * x - 3 * y * y)]
    if L > 3:
        raise ValueError("L <= 3 supported")
    return np.stack(cols, axis=1)


def unit_vectors(n: int, rng: np.random.Generator) -> np.ndarray:
    z = rng.standard_normal((n, 3))
    return z / np.linalg.norm(z, axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# Dense random tensors (chunked so multi-GB fp32 tensors need no fp64 copy)
# ---------------------------------------------------------------------------

def normal(rng: np.random.Generator, shape, dtype, scale: float = 1.0,
           chunk: int = 1 << 24) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=dtype)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        t = rng.standard_normal(b - a)
        if scale != 1.0:
            t *= scale
        out[a:b] = t            # fp64 -> fp32 rounds to nearest even
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# Sub-graphs (selecting edges; used to evaluate sampled rows)
# ---------------------------------------------------------------------------


def subgraph(rowptr: np.ndarray, src: np.ndarray, edges: np.ndarray):
    """Receiver CSR over the same N nodes that keeps only the listed edges
    (sorted ascending, so receivers stay non-decreasing).  Returns
    (rowptr_sub, src_sub, edges)."""
    edges = np.asarray(sorted(set(int(e) for e in edges)), dtype=np.int64)
    N = len(rowptr) - 1
    recv = np.searchsorted(rowptr, edges, side="right") - 1
    counts = np.bincount(recv, minlength=N)
    rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return rp, src[edges].astype(np.int32), edges


def edges_of_rows(rowptr: np.ndarray, rows) -> np.ndarray:
    return np.concatenate([np.arange(rowptr[r], rowptr[r + 1]) for r in rows] + [np.zeros(0, np.int64)])


def _children(seed: int):
    return [np.random.Generator(np.random.PCG64(c))
            for c in np.random.SeedSequence(seed).spawn(_NCHILD)]


def generate(wl: Workload, n_paths: int, out_dim: int, want=("x", "Y", "W", "g"),
             ) -> dict:
    """Inputs of one workload.  n_paths and out_dim describe the W and g shapes
    (they follow from the path list, which this module does not compute)."""
    rngs = _children(wl.seed)
    degrees = wl.degrees if wl.degrees is not None else [wl.degree] * wl.n_nodes
    if wl.one_sender:
        rowptr = np.concatenate([[0], np.cumsum(degrees)]).astype(np.int32)
        src = np.zeros(int(rowptr[-1]), dtype=np.int32)
    else:
        rowptr, src = make_graph(wl.n_nodes, degrees, rngs[_GRAPH], multi=wl.multi)
    E = int(rowptr[-1])
    dt = wl.np_dtype()
    out = {"rowptr": rowptr, "src": src, "N": wl.n_nodes, "E": E}
    if "Y" in want or "vec" in want:
        vec = unit_vectors(E, rngs[_VEC])
        out["vec"] = vec
        full = real_sh_cartesian(max(wl.y_degrees), vec)
        # each Y block holds the harmonics of its degree (whatever parity it is labelled with)
        out["Y"] = np.concatenate([full[:, l * l:(l + 1) ** 2] for l in wl.y_degrees], axis=1).astype(dt)
    if "evec" in want:
        # edge vectors with lengths: the unit vectors above times lengths uniform in [0.5, 5)
        unit = out["vec"] if "vec" in out else unit_vectors(E, _children(wl.seed)[_VEC])
        lrng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(wl.seed).spawn(_NCHILD)[_EXTRA].spawn(100)[99]))
        out["evec"] = (unit * (0.5 + 4.5 * lrng.random((E, 1)))).astype(dt)
    if "pos" in want:
        # atom positions uniform in a 10 x 10 x 10 box (the graph is drawn independently of them)
        prng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(wl.seed).spawn(_NCHILD)[_EXTRA].spawn(100)[98]))
        out["pos"] = (10.0 * prng.random((wl.n_nodes, 3))).astype(dt)
    if "x" in want:
        out["x"] = normal(rngs[_X], (wl.n_nodes, wl.x_dim), dt)
    if "W" in want:
        scale = 1.0 / math.sqrt(n_paths) if wl.w_scale == "inv_sqrt_paths" else 1.0
        out["W"] = normal(rngs[_W], (E, n_paths, wl.U), dt, scale)
    if "g" in want:
        out["g"] = normal(rngs[_G], (wl.n_nodes, out_dim), dt)
    if "v" in want:
        out["v"] = normal(rngs[_V], (wl.n_nodes, wl.x_dim), dt)
    return out


def extra_normal(wl: Workload, shape, k: int = 0) -> np.ndarray:
    """Further N(0,1) tensors (tangents for double-backward tests)."""
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(wl.seed).spawn(_NCHILD)[_EXTRA].spawn(k + 1)[k]))
    return normal(rng, shape, wl.np_dtype())
