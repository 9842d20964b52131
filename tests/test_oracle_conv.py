"""Pins of the oracle's convolution, its VJP and its double backward.

Independent checks only: a dense einsum with one-hot incidence matrices (no CSR
code, no sparse tables), scipy.sparse for the scalar path, rotation and
inversion equivariance, the adjoint identities of a trilinear map, and exact
five-point finite differences (every quantity below is a polynomial of degree
<= 3 along a line, for which the five-point stencil is exact).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import sphere


def _dense_fwd(d, rowptr, src, x, Y, W):
    """out = A_recv^T msg, msg[e] = sum_p C_p(x[src[e]], Y[e]) W[e,p] (dense)."""
    N, E = len(rowptr) - 1, len(src)
    recv = np.repeat(np.arange(N), np.diff(rowptr))
    A_send = np.zeros((E, N)); A_send[np.arange(E), src] = 1
    A_recv = np.zeros((E, N)); A_recv[np.arange(E), recv] = 1
    xs = A_send @ x
    xoff = np.cumsum([0] + [d.U * (2 * l + 1) for l in d.xl])
    ooff = np.cumsum([0] + [d.U * (2 * l + 1) for l in d.out_l])
    out = np.zeros((N, d.out_dim))
    yoff = np.cumsum([0] + [2 * l + 1 for l in d.yl])
    xm = getattr(d, "xm", [d.U] * len(d.xl))
    om = getattr(d, "out_mul", [d.U] * len(d.out_l))
    xoff = np.cumsum([0] + [m * (2 * l + 1) for m, l in zip(xm, d.xl)])
    ooff = np.cumsum([0] + [m * (2 * l + 1) for m, l in zip(om, d.out_l)])
    for p, (i1, iy, l3, ob) in enumerate(d.paths):
        l1, l2 = d.xl[i1], d.yl[iy]
        C = oracle.cg_real(l1, l2, l3)
        xb = xs[:, xoff[i1]:xoff[i1 + 1]].reshape(E, xm[i1], 2 * l1 + 1)
        xb = np.broadcast_to(xb, (E, d.U, 2 * l1 + 1))       # a one-channel block feeds every channel
        yb = Y[:, yoff[iy]:yoff[iy + 1]]
        msg = np.einsum("eua,eb,abc,eu->euc", xb, yb, C, W[:, p, :])
        if om[ob] == 1:
            msg = msg.sum(axis=1, keepdims=True)              # a one-channel output sums the channels
        out[:, ooff[ob]:ooff[ob + 1]] += A_recv.T @ msg.reshape(E, -1)
    return out


def _tiny_graph(rng, N=9, with_dups=True):
    deg = rng.integers(0, 6, size=N)
    deg[2] = 0                                    # an empty row
    rowptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    src = rng.integers(0, N, size=rowptr[-1]).astype(np.int32)   # self-loops, duplicates
    if with_dups and len(src) > 1:
        src[1] = src[0]
    return rowptr, src


def _tiny_inputs(d, rowptr, src, rng):
    N, E = len(rowptr) - 1, len(src)
    x = rng.standard_normal((N, d.x_dim))
    Y = synth.real_sh_cartesian(d.L, synth.unit_vectors(E, rng))
    W = rng.standard_normal((E, d.P, d.U))
    g = rng.standard_normal((N, d.out_dim))
    return x, Y, W, g


DESCS = [
    dict(x_irreps=((3, 0, 1), (3, 1, -1)), y_lmax=2, l3_max=1),
    dict(x_irreps=((2, 0, 1), (2, 1, -1), (2, 2, 1)), y_lmax=3, l3_max=3),
    dict(x_irreps=((2, 3, -1), (2, 1, 1)), y_lmax=3, l3_max=3),
]


def test_path_enumeration_counts_and_order():
    got = {k: oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max).P
           for k, wl in synth.WORKLOADS.items()}
    assert got == {"tiny_fp64": 6, "mace_medium_fp32": 13, "mace_medium_fp64": 13,
                   "mace_large_fp32": 24, "wide_proxy_fp32": 24, "invariant_fp32": 4}
    # invariant outputs: l3 = 0 needs l2 = l1, and p1 (-1)^l1 is even for 0e, 1o, 2e, 3o
    assert oracle.enumerate_paths(synth.WORKLOADS["invariant_fp32"].x_irreps, 3, 0) == [
        (0, 0, 0, 1), (1, 1, 0, 1), (2, 2, 0, 1), (3, 3, 0, 1)]
    en = oracle.enumerate_paths(synth.WORKLOADS["tiny_fp64"].x_irreps, 2, 1)
    # 0e x 0e -> 0e, 0e x 1o -> 1o, 1o x 0e -> 1o, 1o x 1o -> 0e, 1o x 1o -> 1e, 1o x 2e -> 1o
    assert en == [(0, 0, 0, 1), (0, 1, 1, -1), (1, 0, 1, -1), (1, 1, 0, 1), (1, 1, 1, 1),
                  (1, 2, 1, -1)]


def test_sparse_table_sizes():
    d = oracle.Desc(synth.WORKLOADS["mace_medium_fp32"].x_irreps, 3, 3)
    nnz = sum(np.count_nonzero(oracle.cg_real(d.xl[i1], l2, l3)) for i1, l2, l3, _ in d.paths)
    assert nnz == 134
    assert d.out_dim // d.U == 55
    d = oracle.Desc(synth.WORKLOADS["mace_large_fp32"].x_irreps, 3, 3)
    nnz = sum(np.count_nonzero(oracle.cg_real(d.xl[i1], l2, l3)) for i1, l2, l3, _ in d.paths)
    assert nnz == 351
    assert d.out_dim // d.U == 106


@pytest.mark.parametrize("k", range(len(DESCS)))
def test_fwd_matches_dense_einsum(k):
    rng = np.random.default_rng(10 + k)
    d = oracle.Desc(**DESCS[k])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, _ = _tiny_inputs(d, rowptr, src, rng)
    ref = _dense_fwd(d, rowptr, src, x, Y, W)
    got = oracle.fwd(d, rowptr, src, x, Y, W)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    assert not got[2].any()                      # empty receiver row


def test_fwd_shared_output_block_sums_paths():
    """Two paths pointed at one output block are summed into it."""
    rng = np.random.default_rng(20)
    xi = ((2, 1, -1),)
    d_sep = oracle.Desc(xi, 2, paths=[(0, 0, 1, 0), (0, 2, 1, 1)], out_l=[1, 1])
    d_sum = oracle.Desc(xi, 2, paths=[(0, 0, 1, 0), (0, 2, 1, 0)], out_l=[1])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, _ = _tiny_inputs(d_sep, rowptr, src, rng)
    a = oracle.fwd(d_sep, rowptr, src, x, Y, W)
    b = oracle.fwd(d_sum, rowptr, src, x, Y, W)
    assert np.allclose(b, a[:, :6] + a[:, 6:], atol=1e-13)
    assert np.allclose(b, _dense_fwd(d_sum, rowptr, src, x, Y, W), atol=1e-13)


def test_fwd_scalar_path_is_weighted_spmm():
    import scipy.sparse as sp
    rng = np.random.default_rng(30)
    U = 5
    d = oracle.Desc(((U, 0, 1),), 0, 0)
    assert d.paths == [(0, 0, 0, 0)]
    rowptr, src = _tiny_graph(rng, N=12)
    N, E = len(rowptr) - 1, len(src)
    x = rng.standard_normal((N, U))
    Y = rng.standard_normal((E, 1))
    W = rng.standard_normal((E, 1, U))
    got = oracle.fwd(d, rowptr, src, x, Y, W)
    for u in range(U):
        A = sp.csr_matrix((Y[:, 0] * W[:, 0, u], src, rowptr), shape=(N, N))
        assert np.allclose(got[:, u], A @ x[:, u], atol=1e-13)


def test_fwd_rows_subset():
    rng = np.random.default_rng(40)
    d = oracle.Desc(**DESCS[1])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, _ = _tiny_inputs(d, rowptr, src, rng)
    full = oracle.fwd(d, rowptr, src, x, Y, W)
    rows = np.array([5, 0, 2])
    assert np.array_equal(oracle.fwd(d, rowptr, src, x, Y, W, rows=rows), full[rows])


@pytest.mark.parametrize("k", range(len(DESCS)))
def test_fwd_rotation_equivariance(k):
    rng = np.random.default_rng(50 + k)
    d = oracle.Desc(**DESCS[k])
    rowptr, src = _tiny_graph(rng)
    N, E = len(rowptr) - 1, len(src)
    vec = synth.unit_vectors(E, rng)
    x = rng.standard_normal((N, d.x_dim))
    W = rng.standard_normal((E, d.P, d.U))
    ang = tuple(rng.uniform(0.1, 3.0, 3))
    R = sphere.rotation(*ang)
    Dx = sphere.block_diag_irreps([(d.U, l) for l in d.xl], *ang)
    Do = sphere.block_diag_irreps([(d.U, l) for l in d.out_l], *ang)
    Y = synth.real_sh_cartesian(d.L, vec)
    YR = synth.real_sh_cartesian(d.L, vec @ R.T)          # rotated edge vectors
    out = oracle.fwd(d, rowptr, src, x, Y, W)
    outR = oracle.fwd(d, rowptr, src, x @ Dx.T, YR, W)
    assert np.abs(outR - out @ Do.T).max() < 1e-11 * np.abs(out).max()


@pytest.mark.parametrize("k", range(len(DESCS)))
def test_fwd_inversion_parity(k):
    rng = np.random.default_rng(60 + k)
    d = oracle.Desc(**DESCS[k])
    rowptr, src = _tiny_graph(rng)
    E = len(src)
    x, _, W, _ = _tiny_inputs(d, rowptr, src, rng)
    vec = synth.unit_vectors(E, rng)
    Y, Yinv = synth.real_sh_cartesian(d.L, vec), synth.real_sh_cartesian(d.L, -vec)
    px = np.concatenate([np.full(d.U * (2 * l + 1), p) for (_, l, p) in d.x_irreps])
    en = oracle.enumerate_paths(d.x_irreps, d.L, DESCS[k]["l3_max"])
    po = np.concatenate([np.full(d.U * (2 * l3 + 1), p3) for (_, _, l3, p3) in en])
    out = oracle.fwd(d, rowptr, src, x, Y, W)
    outI = oracle.fwd(d, rowptr, src, x * px, Yinv, W)
    assert np.allclose(outI, out * po, atol=1e-12)


# ---------------------------------------------------------------------------
# VJP
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", range(len(DESCS)))
def test_vjp_adjoint_identities(k):
    rng = np.random.default_rng(70 + k)
    d = oracle.Desc(**DESCS[k])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, g = _tiny_inputs(d, rowptr, src, rng)
    f = oracle.fwd(d, rowptr, src, x, Y, W)
    gx, gY, gW = oracle.bwd(d, rowptr, src, x, Y, W, g)
    L = np.vdot(g, f)
    for grad, arg in ((gx, x), (gY, Y), (gW, W)):
        assert np.vdot(grad, arg) == pytest.approx(L, rel=1e-12, abs=1e-12)


def _five_point(fn, h=0.5):
    return (8 * (fn(h) - fn(-h)) - (fn(2 * h) - fn(-2 * h))) / (12 * h)


@pytest.mark.parametrize("k", range(len(DESCS)))
def test_vjp_is_gradient_along_mixed_direction(k):
    rng = np.random.default_rng(80 + k)
    d = oracle.Desc(**DESCS[k])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, g = _tiny_inputs(d, rowptr, src, rng)
    dx, dY, dW = (rng.standard_normal(a.shape) for a in (x, Y, W))

    def loss(t):
        return np.vdot(g, oracle.fwd(d, rowptr, src, x + t * dx, Y + t * dY, W + t * dW))

    gx, gY, gW = oracle.bwd(d, rowptr, src, x, Y, W, g)
    pred = np.vdot(gx, dx) + np.vdot(gY, dY) + np.vdot(gW, dW)
    assert _five_point(loss) == pytest.approx(pred, rel=1e-10)
    # each argument alone: the loss is linear in it, so a one-sided difference is exact
    for grad, arg, dd, which in ((gx, x, dx, 0), (gY, Y, dY, 1), (gW, W, dW, 2)):
        args = [x, Y, W]
        args[which] = arg + dd
        delta = np.vdot(g, oracle.fwd(d, rowptr, src, *args)) - np.vdot(
            g, oracle.fwd(d, rowptr, src, x, Y, W))
        assert delta == pytest.approx(np.vdot(grad, dd), rel=1e-10)


def test_vjp_subsets_match_full():
    rng = np.random.default_rng(90)
    d = oracle.Desc(**DESCS[1])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, g = _tiny_inputs(d, rowptr, src, rng)
    gx, gY, gW = oracle.bwd(d, rowptr, src, x, Y, W, g)
    e = np.array([3, 0, len(src) - 1])
    sW, sY = oracle.bwd_edges(d, rowptr, src, x, Y, W, g, edges=e)
    assert np.array_equal(sW, gW[e]) and np.array_equal(sY, gY[e])
    s = np.array([4, 1])
    assert np.array_equal(oracle.bwd_gx(d, rowptr, src, Y, W, g, senders=s), gx[s])


def test_vjp_gradient_rotation_equivariance():
    """gx rotates like x and gY like Y when g rotates like the output."""
    rng = np.random.default_rng(95)
    d = oracle.Desc(**DESCS[1])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, g = _tiny_inputs(d, rowptr, src, rng)
    ang = (0.3, 2.1, -0.8)
    Dx = sphere.block_diag_irreps([(d.U, l) for l in d.xl], *ang)
    Do = sphere.block_diag_irreps([(d.U, l) for l in d.out_l], *ang)
    DY = sphere.block_diag_irreps([(1, l) for l in range(d.L + 1)], *ang)
    gx, gY, gW = oracle.bwd(d, rowptr, src, x, Y, W, g)
    gx2, gY2, gW2 = oracle.bwd(d, rowptr, src, x @ Dx.T, Y @ DY.T, W, g @ Do.T)
    assert np.allclose(gx2, gx @ Dx.T, atol=1e-11)
    assert np.allclose(gY2, gY @ DY.T, atol=1e-11)
    assert np.allclose(gW2, gW, atol=1e-11)


# ---------------------------------------------------------------------------
# Double backward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", range(len(DESCS)))
def test_dbwd_matches_finite_differences_of_vjp(k):
    rng = np.random.default_rng(100 + k)
    d = oracle.Desc(**DESCS[k])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, g = _tiny_inputs(d, rowptr, src, rng)
    ggx, ggY, ggW = (rng.standard_normal(a.shape) for a in (x, Y, W))
    res = oracle.dbwd(d, rowptr, src, x, Y, W, g, ggx, ggY, ggW)

    def S(xx, YY, WW, gg):
        gx, gY, gW = oracle.bwd(d, rowptr, src, xx, YY, WW, gg)
        return np.vdot(ggx, gx) + np.vdot(ggY, gY) + np.vdot(ggW, gW)

    base = (x, Y, W, g)
    names = ("dx", "dY", "dW", "dg")
    dirs = [rng.standard_normal(a.shape) for a in base]
    # each argument separately
    for i, name in enumerate(names):
        def line(t, i=i):
            a = list(base)
            a[i] = base[i] + t * dirs[i]
            return S(*a)
        assert _five_point(line) == pytest.approx(np.vdot(res[name], dirs[i]), rel=1e-9, abs=1e-9)
    # all at once
    def line_all(t):
        return S(*(b + t * v for b, v in zip(base, dirs)))
    pred = sum(np.vdot(res[n], v) for n, v in zip(names, dirs))
    assert _five_point(line_all) == pytest.approx(pred, rel=1e-9)


def test_hvp_tangent_on_x_only():
    """With only ggx set: dx is exactly zero, dg = f(v, Y, W)."""
    rng = np.random.default_rng(110)
    d = oracle.Desc(**DESCS[1])
    rowptr, src = _tiny_graph(rng)
    x, Y, W, g = _tiny_inputs(d, rowptr, src, rng)
    v = rng.standard_normal(x.shape)
    res = oracle.dbwd(d, rowptr, src, x, Y, W, g, ggx=v)
    assert not res["dx"].any()
    assert np.array_equal(res["dg"], oracle.fwd(d, rowptr, src, v, Y, W))
    rows, edges, senders = np.array([1, 7]), np.array([0, 4]), np.array([3])
    sub = oracle.dbwd(d, rowptr, src, x, Y, W, g, ggx=v, rows=rows, edges=edges, senders=senders)
    assert np.array_equal(sub["dg"], res["dg"][rows])
    assert np.array_equal(sub["dY"], res["dY"][edges])
    assert np.array_equal(sub["dW"], res["dW"][edges])


# ---------------------------------------------------------------------------
# Sender CSR
# ---------------------------------------------------------------------------

def test_sender_csr_is_stable_counting_sort():
    rng = np.random.default_rng(120)
    N = 50
    src = rng.integers(0, N, size=700).astype(np.int32)
    src[src == 7] = 8                                   # a sender with no edges
    srowptr, sperm = oracle.sender_csr(N, src)
    assert np.array_equal(sperm, np.argsort(src, kind="stable"))
    assert np.array_equal(srowptr, np.concatenate([[0], np.cumsum(np.bincount(src, minlength=N))]))
    assert srowptr[7] == srowptr[8]
    assert np.all(np.diff(src[sperm]) >= 0)
    assert np.array_equal(np.sort(sperm), np.arange(len(src)))
    e0, e1 = oracle.sender_csr(0, np.zeros(0, dtype=np.int32))
    assert e0.tolist() == [0] and len(e1) == 0


def test_generator_graph_properties():
    wl = synth.WORKLOADS["tiny_fp64"]
    d = oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max)
    inp = synth.generate(wl, d.P, d.out_dim)
    rowptr, src = inp["rowptr"], inp["src"]
    assert rowptr[0] == 0 and rowptr[-1] == wl.n_edges == 1024
    assert np.all(np.diff(rowptr) == 16)
    for r in range(wl.n_nodes):
        row = src[rowptr[r]:rowptr[r + 1]]
        assert np.all(np.diff(row) > 0) and r not in row
    assert inp["W"].shape == (1024, 6, 8) and inp["x"].dtype == np.float64
    again = synth.generate(wl, d.P, d.out_dim)
    assert np.array_equal(again["W"], inp["W"]) and np.array_equal(again["src"], src)


# ---------------------------------------------------------------------------
# Y given as a list of irreps (any degrees, in any order, with either parity)
# ---------------------------------------------------------------------------

Y_SUBSET = ((1, 2, 1), (1, 0, 1), (1, 1, 1))      # 2e + 0e + 1e: no degree 3, a pseudovector, unsorted


def test_path_enumeration_with_y_irreps():
    # x = 1o; Y = 0e + 1e: 1o x 0e -> 1o; 1o x 1e -> 0o, 1o, 2o (parity -1 * +1)
    en = oracle.enumerate_paths(((4, 1, -1),), 0, 3, y_irreps=((1, 0, 1), (1, 1, 1)))
    assert en == [(0, 0, 1, -1), (0, 1, 0, -1), (0, 1, 1, -1), (0, 1, 2, -1)]
    # the default Y is the harmonics 0e, 1o, 2e, 3o: the same list as y_lmax alone
    x = synth.WORKLOADS["mace_large_fp32"].x_irreps
    assert oracle.enumerate_paths(x, 3, 3) == oracle.enumerate_paths(
        x, 0, 3, y_irreps=((1, 0, 1), (1, 1, -1), (1, 2, 1), (1, 3, -1)))
    d = oracle.Desc(((3, 0, 1), (3, 1, -1)), 0, 2, y_irreps=Y_SUBSET)
    assert d.y_dim == 9 and d.yoff == [0, 5, 6]
    # 0e x (2e, 0e, 1e) -> 2, 0, 1; 1o x 2e -> 1, 2 (l3 <= 2); 1o x 0e -> 1; 1o x 1e -> 0, 1, 2
    assert [d.path_l2(p) for p in range(d.P)] == [2, 0, 1, 2, 2, 0, 1, 1, 1]
    assert [p[2] for p in d.paths] == [2, 0, 1, 1, 2, 1, 0, 1, 2]


def test_fwd_with_y_irreps_matches_dense_einsum():
    rng = np.random.default_rng(40)
    d = oracle.Desc(((3, 0, 1), (3, 1, -1), (3, 2, 1)), 0, 3, y_irreps=Y_SUBSET)
    rowptr, src = _tiny_graph(rng)
    N, E = len(rowptr) - 1, len(src)
    x = rng.standard_normal((N, d.x_dim))
    Y = rng.standard_normal((E, d.y_dim))
    W = rng.standard_normal((E, d.P, d.U))
    ref = _dense_fwd(d, rowptr, src, x, Y, W)
    got = oracle.fwd(d, rowptr, src, x, Y, W)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_y_subset_equals_full_y_on_the_matching_paths():
    """Y = 2e + 0e (a subset, reordered) gives what Y = 0e + 1o + 2e gives on the paths of
    degrees 0 and 2, whatever the degree-1 columns hold; every output of the VJP too."""
    rng = np.random.default_rng(41)
    xi = ((2, 1, -1), (2, 2, 1))
    sub = oracle.Desc(xi, 0, 3, y_irreps=((1, 2, 1), (1, 0, 1)))
    full_all = oracle.Desc(xi, 2, 3)
    # the full descriptor restricted to the subset's paths, in the subset's order
    to_full = {0: 2, 1: 0}
    paths = [(i1, to_full[iy], l3, k) for k, (i1, iy, l3, _) in enumerate(sub.paths)]
    full = oracle.Desc(xi, 2, 3, paths=paths, out_l=sub.out_l)
    assert full.P == sub.P < full_all.P
    rowptr, src = _tiny_graph(rng)
    N, E = len(rowptr) - 1, len(src)
    x = rng.standard_normal((N, sub.x_dim))
    Ys = rng.standard_normal((E, sub.y_dim))
    Yf = rng.standard_normal((E, full.y_dim))        # degree-1 columns: anything
    Yf[:, 4:9], Yf[:, 0:1] = Ys[:, 0:5], Ys[:, 5:6]
    W = rng.standard_normal((E, sub.P, sub.U))
    g = rng.standard_normal((N, sub.out_dim))
    assert np.allclose(oracle.fwd(sub, rowptr, src, x, Ys, W), oracle.fwd(full, rowptr, src, x, Yf, W), atol=1e-13)
    gs, gf = oracle.bwd(sub, rowptr, src, x, Ys, W, g), oracle.bwd(full, rowptr, src, x, Yf, W, g)
    assert np.allclose(gs[0], gf[0], atol=1e-13) and np.allclose(gs[2], gf[2], atol=1e-13)
    assert np.allclose(gs[1][:, 0:5], gf[1][:, 4:9], atol=1e-13)
    assert np.allclose(gs[1][:, 5:6], gf[1][:, 0:1], atol=1e-13)
    assert not gf[1][:, 1:4].any()                   # no path uses degree 1


def test_vjp_adjoint_with_y_irreps():
    """<g, f(x, Y, W)> = <gx, x> = <gY, Y> = <gW, W> with a Y subset (trilinearity)."""
    rng = np.random.default_rng(42)
    d = oracle.Desc(((3, 0, 1), (3, 1, -1)), 0, 3, y_irreps=Y_SUBSET)
    rowptr, src = _tiny_graph(rng)
    N, E = len(rowptr) - 1, len(src)
    x, Y = rng.standard_normal((N, d.x_dim)), rng.standard_normal((E, d.y_dim))
    W, g = rng.standard_normal((E, d.P, d.U)), rng.standard_normal((N, d.out_dim))
    f = np.vdot(g, oracle.fwd(d, rowptr, src, x, Y, W))
    gx, gY, gW = oracle.bwd(d, rowptr, src, x, Y, W, g)
    for a, b in ((gx, x), (gY, Y), (gW, W)):
        assert abs(np.vdot(a, b) - f) <= 1e-12 * max(1.0, abs(f))


# ---------------------------------------------------------------------------
# UVW products that reduce to the channel-wise one: a one-channel x block broadcast
# against the U channels, and one-channel output blocks that sum the channels
# ---------------------------------------------------------------------------

def _mixed(seed, U=3):
    rng = np.random.default_rng(seed)
    rowptr, src = _tiny_graph(rng)
    N, E = len(rowptr) - 1, len(src)
    return rng, rowptr, src, N, E


def _expand_x(d_one, d_full, x):
    """x of d_one (one-channel blocks) as the x of d_full (those blocks with U channels),
    every channel a copy."""
    out = []
    o = 0
    for (m, l, _p) in d_one.x_irreps:
        n = 2 * l + 1
        blk = x[:, o:o + m * n].reshape(len(x), m, n)
        out.append(np.broadcast_to(blk, (len(x), d_full.U, n)).reshape(len(x), -1))
        o += m * n
    return np.concatenate(out, axis=1)


def _fold_x(d_one, d_full, gx_full):
    """The gradient of d_full's x folded back onto d_one's layout: summed over the channels
    of the blocks that d_one has with one channel."""
    out = []
    o = 0
    for (m, l, _p) in d_one.x_irreps:
        n = 2 * l + 1
        blk = gx_full[:, o:o + d_full.U * n].reshape(len(gx_full), d_full.U, n)
        out.append((blk.sum(axis=1, keepdims=True) if m == 1 else blk).reshape(len(gx_full), -1))
        o += d_full.U * n
    return np.concatenate(out, axis=1)


def test_one_channel_x_is_the_channel_wise_product_of_its_copies():
    rng, rowptr, src, N, E = _mixed(90)
    one = oracle.Desc(((1, 1, -1), (3, 0, 1)), 2, 2)
    full = oracle.Desc(((3, 1, -1), (3, 0, 1)), 2, 2)
    assert one.P == full.P and one.out_dim == full.out_dim and one.x_dim == 3 + 3
    x = rng.standard_normal((N, one.x_dim))
    Y = synth.real_sh_cartesian(2, synth.unit_vectors(E, rng))
    W = rng.standard_normal((E, one.P, one.U))
    g = rng.standard_normal((N, one.out_dim))
    xf = _expand_x(one, full, x)
    assert np.allclose(oracle.fwd(one, rowptr, src, x, Y, W), oracle.fwd(full, rowptr, src, xf, Y, W), atol=1e-13)
    a, b = oracle.bwd(one, rowptr, src, x, Y, W, g), oracle.bwd(full, rowptr, src, xf, Y, W, g)
    assert np.allclose(a[0], _fold_x(one, full, b[0]), atol=1e-13)        # gx: a sum over the copies
    assert np.allclose(a[1], b[1], atol=1e-13) and np.allclose(a[2], b[2], atol=1e-13)
    assert np.allclose(oracle.fwd(one, rowptr, src, x, Y, W), _dense_fwd(one, rowptr, src, x, Y, W), atol=1e-13)


def test_one_channel_output_is_the_sum_of_the_channel_wise_outputs():
    rng, rowptr, src, N, E = _mixed(91)
    xi = ((3, 0, 1), (3, 1, -1))
    base = oracle.Desc(xi, 2, 2)
    summed = [1 if l3 % 2 == 0 else base.U for l3 in base.out_l]            # the even-degree outputs summed
    one = oracle.Desc(xi, 2, 2, paths=base.paths, out_l=base.out_l, out_mul=summed)
    assert one.out_dim < base.out_dim
    x = rng.standard_normal((N, one.x_dim))
    Y = synth.real_sh_cartesian(2, synth.unit_vectors(E, rng))
    W = rng.standard_normal((E, one.P, one.U))
    out_b = oracle.fwd(base, rowptr, src, x, Y, W)
    out_o = oracle.fwd(one, rowptr, src, x, Y, W)
    # fold base's output onto one's layout, and broadcast one's cotangent onto base's layout
    fold, g_o = [], rng.standard_normal((N, one.out_dim))
    g_b = []
    ob = oo = 0
    for m, l in zip(summed, base.out_l):
        n = 2 * l + 1
        blk = out_b[:, ob:ob + base.U * n].reshape(N, base.U, n)
        fold.append((blk.sum(axis=1) if m == 1 else blk.reshape(N, -1)))
        gblk = g_o[:, oo:oo + m * n].reshape(N, m, n)
        g_b.append(np.broadcast_to(gblk, (N, base.U, n)).reshape(N, -1))
        ob += base.U * n
        oo += m * n
    assert np.allclose(out_o, np.concatenate(fold, axis=1), atol=1e-13)
    assert np.allclose(out_o, _dense_fwd(one, rowptr, src, x, Y, W), atol=1e-13)
    a = oracle.bwd(one, rowptr, src, x, Y, W, g_o)
    b = oracle.bwd(base, rowptr, src, x, Y, W, np.concatenate(g_b, axis=1))
    for u, v in zip(a, b):
        assert np.allclose(u, v, atol=1e-12)


def test_mixed_multiplicities_adjoint_and_dense():
    rng, rowptr, src, N, E = _mixed(92, U=4)
    d = oracle.Desc(((1, 0, 1), (4, 1, -1), (1, 2, 1)), 3, 3)
    om = [1 if k % 3 == 0 else d.U for k in range(len(d.out_l))]
    d = oracle.Desc(((1, 0, 1), (4, 1, -1), (1, 2, 1)), 3, 3, paths=d.paths, out_l=d.out_l, out_mul=om)
    x, Y = rng.standard_normal((N, d.x_dim)), rng.standard_normal((E, d.y_dim))
    W, g = rng.standard_normal((E, d.P, d.U)), rng.standard_normal((N, d.out_dim))
    out = oracle.fwd(d, rowptr, src, x, Y, W)
    assert np.abs(out - _dense_fwd(d, rowptr, src, x, Y, W)).max() <= 1e-12 * np.abs(out).max()
    f = np.vdot(g, out)
    gx, gY, gW = oracle.bwd(d, rowptr, src, x, Y, W, g)
    for a, b in ((gx, x), (gY, Y), (gW, W)):
        assert abs(np.vdot(a, b) - f) <= 1e-12 * max(1.0, abs(f))


def test_output_irreps_collect_the_paths_of_their_irrep():
    # 1o x (0e + 1o + 2e) up to l3 = 1: 1o x 0e -> 1o, 1o x 1o -> 0e and 1e, 1o x 2e -> 1o;
    # given outputs 1o and 0e (one channel), the two 1o paths add into block 0, the 0e
    # path into block 1, and the 1e path is not part of the product
    d = oracle.Desc(((4, 1, -1),), 2, 1, out_irreps=((4, 1, -1), (1, 0, 1)))
    assert d.paths == [(0, 0, 1, 0), (0, 1, 0, 1), (0, 2, 1, 0)]
    assert d.out_l == [1, 0] and d.out_mul == [4, 1] and d.out_dim == 4 * 3 + 1
