"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Small and medium problems are compared element by element on every output.
The full 5,000-node / 280,000-edge workloads run in the same launch shape the
benchmark times and are also compared on every element, except the multi-GB
wide proxy, which is compared on sampled rows (receivers for the forward, edges
for the W and Y gradients, senders for the x gradient) that the oracle evaluates
on the sub-graph of exactly those edges.  Bound: relative L2 per output tensor
<= 1e-5 (fp32) or 1e-12 (fp64); integer outputs bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import RTOL, edges_of_rows, inputs, oracle_desc, plan_for, rel_l2, sample, subgraph, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


W_ = synth.WORKLOADS
# Reduced versions of the named workloads (full comparison): several receivers'
# worth of edge tiles with a ragged tail (degree 56 = 32 + 24).
REDUCED = {
    "tiny_fp64": W_["tiny_fp64"],
    "mace_medium_fp32": W_["mace_medium_fp32"].scaled(n_nodes=240),
    "mace_medium_fp64": W_["mace_medium_fp64"].scaled(n_nodes=240),
    "mace_large_fp32": W_["mace_large_fp32"].scaled(n_nodes=160),
    "wide_proxy_fp32": W_["wide_proxy_fp32"].scaled(n_nodes=96),
    "invariant_fp32": W_["invariant_fp32"].scaled(n_nodes=200),
}
_rng = np.random.default_rng(77)
_deg = _rng.integers(0, 121, size=150)
_deg[[0, 7, 149]] = 0
_multi_deg = np.random.default_rng(78).integers(0, 41, size=110)
_multi_deg[[0, 13, 59, 60, 75]] = 0
_multi_deg = tuple(int(v) for v in _multi_deg)
EDGE_CASES = {
    # U = 96: a full 64-lane wave plus a half-empty one; degrees 0..120 with empty rows
    "ragged_u96_f32": synth.Workload("ragged_u96_f32", 150, 0, synth._irr("96x0e+96x1o+96x2e"), 3, 3,
                                     "f32", "unit", 31, degrees=tuple(int(v) for v in _deg)),
    # one channel, an l=3 x block, fp64
    "u1_l3_f64": synth.Workload("u1_l3_f64", 40, 9, synth._irr("1x3o+1x1e"), 3, 3, "f64", "unit", 32),
    # U = 8 with Y degrees 0..1 only (padded lane reduction) and outputs up to l=2
    "u8_l1_f32": synth.Workload("u8_l1_f32", 50, 12, synth._irr("8x0e+8x1o+8x2e"), 1, 2, "f32", "unit", 33),
    # the largest multiplicity: 16 waves per workgroup (register-capped kernels)
    "u1024_f32": synth.Workload("u1024_f32", 24, 5, synth._irr("1024x0e+1024x1o"), 2, 2, "f32", "unit", 34),
    # one hub receiver with 3,000 distinct senders (a long edge loop, 94 Y tiles) among
    # 3,099 receivers of one edge each
    "hub_u32_f32": synth.Workload("hub_u32_f32", 3100, 0, synth._irr("32x0e+32x1o"), 3, 3, "f32", "unit", 35,
                                  degrees=(3000,) + (1,) * 3099),
    # multigraphs: senders drawn with replacement from all nodes, so rows hold self-loops
    # (out[r] and gx[r] of the same node in one edge) and repeated (s, r) edges; in-degrees
    # 0..40 with empty rows; one full wave (U = 64) in fp32, a partial wave (U = 40) in fp64
    "multi_u64_f32": synth.Workload("multi_u64_f32", 60, 0, synth._irr("64x0e+64x1o+64x2e"), 3, 3, "f32", "unit",
                                    36, degrees=_multi_deg[:60], multi=True),
    "multi_u40_f64": synth.Workload("multi_u40_f64", 50, 0, synth._irr("40x0e+40x1o"), 2, 2, "f64", "unit", 37,
                                    degrees=_multi_deg[60:], multi=True),
    # Y given as irreps: unsorted degrees with a pseudovector block (2e + 0e + 1e) in fp32,
    # and the odd degrees only (1o + 3o) in fp64
    "ysub_u48_f32": synth.Workload("ysub_u48_f32", 80, 20, synth._irr("48x0e+48x1o+48x2e"), 0, 3, "f32", "unit", 38,
                                   y_irreps=synth._irr("1x2e+1x0e+1x1e")),
    "ysub_u16_f64": synth.Workload("ysub_u16_f64", 60, 14, synth._irr("16x0e+16x1o+16x2e"), 0, 3, "f64", "unit", 39,
                                   y_irreps=synth._irr("1x1o+1x3o")),
}
MULTI = ["multi_u64_f32", "multi_u40_f64"]
YSUB = ["ysub_u48_f32", "ysub_u16_f64"]
SMALL = {**REDUCED, **EDGE_CASES}


def _dev_inputs(inp, dt):
    d = {}
    for k in ("rowptr", "src"):
        d[k] = to_dev(inp[k])
    for k in ("x", "Y", "W", "g", "v"):
        if k in inp:
            d[k] = to_dev(inp[k])
    return d


def _case(name):
    wl = SMALL[name]
    d, inp = inputs(wl, want=("x", "Y", "W", "g", "v"))
    return wl, d, inp, _dev_inputs(inp, wl.dtype), plan_for(wl)


@pytest.mark.parametrize("name", list(SMALL))
def test_fwd_parity(name):
    wl, d, inp, g, plan = _case(name)
    print(f"[fwd] {name} N={wl.n_nodes} E={inp['E']}", flush=True)
    out = oeq.oeq_tp_conv_fwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"])
    torch.cuda.synchronize()
    ref = oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"])
    assert rel_l2(out.cpu().numpy(), ref) <= RTOL[wl.dtype]
    deg = np.diff(inp["rowptr"])
    assert not out.cpu().numpy()[deg == 0].any()          # receivers without edges


# The forward's other forms on every small case: the one the planner does not choose by
# default (CG literals for fp64 and for four or more channel chunks, Y-contracted rows in
# LDS otherwise; tiles of 64 edges, so the hub's 3,000 edges run 47 tiles), and workgroups
# of one channel chunk in an XCD-affine order (U = 96: a half-empty second chunk; U = 1024:
# 16 chunks, the mapping for chunk counts that do not divide 8; U = 1: one chunk).
def _tile_form_default(wl):
    return wl.dtype == "f64" or wl.x_irreps[0][0] > 192


OTHER_FORMS = [(n, {"OEQ_FWD_LDS": "0" if _tile_form_default(SMALL[n]) else "1"}) for n in SMALL] + [
    (n, {"OEQ_FWD_XCD": "1"}) for n in ("ragged_u96_f32", "u1024_f32", "hub_u32_f32", "u1_l3_f64")]


@pytest.mark.parametrize("name,env", OTHER_FORMS,
                         ids=[f"{n}-{'-'.join(f'{k[4:]}{v}' for k, v in e.items())}" for n, e in OTHER_FORMS])
def test_fwd_parity_other_forms(name, env):
    wl = SMALL[name]
    d, inp = inputs(wl, want=("x", "Y", "W"))
    g = _dev_inputs(inp, wl.dtype)
    plan = plan_for(wl, env)
    print(f"[fwd form] {name} {env} N={wl.n_nodes} E={inp['E']}", flush=True)
    out = oeq.oeq_tp_conv_fwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"])
    torch.cuda.synchronize()
    ref = oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"])
    assert rel_l2(out.cpu().numpy(), ref) <= RTOL[wl.dtype]
    deg = np.diff(inp["rowptr"])
    assert not out.cpu().numpy()[deg == 0].any()


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("name", list(SMALL))
def test_bwd_parity(name, mode):
    wl, d, inp, g, plan = _case(name)
    print(f"[bwd] {name} {mode} N={wl.n_nodes} E={inp['E']}", flush=True)
    gx, gY, gW = oeq.oeq_tp_conv_bwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], mode=mode)
    torch.cuda.synchronize()
    rx, rY, rW = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"])
    tol = RTOL[wl.dtype]
    assert rel_l2(gx.cpu().numpy(), rx) <= tol
    assert rel_l2(gY.cpu().numpy(), rY) <= tol
    assert rel_l2(gW.cpu().numpy(), rW) <= tol


@pytest.mark.parametrize("name", ["mace_medium_fp32", "u8_l1_f32"])
def test_bwd_partial_outputs(name):
    """Requesting a subset of the gradients gives the same values for it."""
    wl, d, inp, g, plan = _case(name)
    full = oeq.oeq_tp_conv_bwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"])
    for need in (("Y",), ("W",), ("x",), ("Y", "W")):
        part = oeq.oeq_tp_conv_bwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], need=need)
        for k, a, b in zip(("x", "Y", "W"), full, part):
            if k in need:
                assert rel_l2(b.cpu().numpy(), a.cpu().numpy()) <= RTOL[wl.dtype]
            else:
                assert b is None


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("name", ["mace_large_fp32", "wide_proxy_fp32", "ragged_u96_f32", "tiny_fp64", "u1024_f32",
                                  "hub_u32_f32"] + MULTI + YSUB)
def test_hvp_parity(name, mode):
    """Double backward with a tangent on x only (the HVP of the workloads)."""
    wl, d, inp, g, plan = _case(name)
    print(f"[hvp] {name} {mode}", flush=True)
    res = oeq.oeq_tp_conv_dbwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], gg_x=g["v"],
                               mode=mode)
    torch.cuda.synchronize()
    ref = oracle.dbwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"], ggx=inp["v"])
    tol = RTOL[wl.dtype]
    assert not res["x"].any().item()                       # exactly zero without Y or W tangents
    assert rel_l2(res["Y"].cpu().numpy(), ref["dY"]) <= tol
    assert rel_l2(res["W"].cpu().numpy(), ref["dW"]) <= tol
    assert rel_l2(res["grad_out"].cpu().numpy(), ref["dg"]) <= tol


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("mask", [1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("name", ["u8_l1_f32", "u1_l3_f64", "ragged_u96_f32", "u1024_f32"] + MULTI + YSUB)
def test_dbwd_all_tangents(name, mask, mode):
    wl, d, inp, g, plan = _case(name)
    tx = synth.extra_normal(wl, inp["x"].shape, 0)
    tY = synth.extra_normal(wl, inp["Y"].shape, 1)
    tW = synth.extra_normal(wl, inp["W"].shape, 2)
    gx_ = to_dev(tx) if mask & 1 else None
    gY_ = to_dev(tY) if mask & 2 else None
    gW_ = to_dev(tW) if mask & 4 else None
    res = oeq.oeq_tp_conv_dbwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], gg_x=gx_,
                               gg_Y=gY_, gg_W=gW_, mode=mode)
    torch.cuda.synchronize()
    ref = oracle.dbwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"],
                      ggx=tx if mask & 1 else None, ggY=tY if mask & 2 else None, ggW=tW if mask & 4 else None)
    tol = RTOL[wl.dtype]
    for k, rk in (("x", "dx"), ("Y", "dY"), ("W", "dW"), ("grad_out", "dg")):
        got = res[k].cpu().numpy()
        if not np.any(ref[rk]):
            assert not got.any(), k
        else:
            assert rel_l2(got, ref[rk]) <= tol, k


def test_empty_graph_and_no_nodes():
    wl = W_["mace_medium_fp32"].scaled(n_nodes=20, degree=0)
    d, inp = inputs(wl)
    g = _dev_inputs(inp, wl.dtype)
    plan = plan_for(wl)
    assert inp["E"] == 0
    out = oeq.oeq_tp_conv_fwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"])
    gx, gY, gW = oeq.oeq_tp_conv_bwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"])
    res = oeq.oeq_tp_conv_dbwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], gg_x=g["x"],
                               mode="deterministic")
    torch.cuda.synchronize()
    assert out.shape == (20, plan.out_dim) and not out.any().item()
    assert not gx.any().item() and gY.shape == (0, 16) and gW.shape == (0, plan.n_paths, plan.U)
    assert not res["x"].any().item() and not res["grad_out"].any().item()
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    x0 = torch.zeros(0, plan.x_dim, device="cuda")
    y0 = torch.zeros(0, 16, device="cuda")
    w0 = torch.zeros(0, plan.n_paths, plan.U, device="cuda")
    assert oeq.oeq_tp_conv_fwd(plan, z, e, x0, y0, w0).shape == (0, plan.out_dim)


def test_sender_csr_bit_exact():
    wl = SMALL["ragged_u96_f32"]
    _, inp = inputs(wl, want=())
    srp, spm = oeq.oeq_sender_csr(to_dev(inp["src"]), wl.n_nodes)
    r_srp, r_spm = oracle.sender_csr(wl.n_nodes, inp["src"])
    assert np.array_equal(srp.cpu().numpy(), r_srp)
    assert np.array_equal(spm.cpu().numpy(), r_spm)
    big = W_["mace_medium_fp32"]
    _, inp = inputs(big, want=())
    srp, spm = oeq.oeq_sender_csr(to_dev(inp["src"]), big.n_nodes)
    r_srp, r_spm = oracle.sender_csr(big.n_nodes, inp["src"])
    assert np.array_equal(srp.cpu().numpy(), r_srp) and np.array_equal(spm.cpu().numpy(), r_spm)


def test_csr_check():
    wl = SMALL["ragged_u96_f32"]
    _, inp = inputs(wl, want=())
    rp, src = to_dev(inp["rowptr"]), to_dev(inp["src"])
    oeq.oeq_csr_check(rp, src)
    bad = src.clone()
    bad[3] = wl.n_nodes
    with pytest.raises(oeq.OeqError):
        oeq.oeq_csr_check(rp, bad)


@pytest.mark.parametrize("name", ["mace_medium_fp32", "mace_medium_fp64", "ragged_u96_f32", "hub_u32_f32"] + MULTI)
def test_bitwise_repeatable(name):
    """The forward and the deterministic backward are bitwise repeatable; the
    atomic backward agrees with them within the tolerance."""
    wl, d, inp, g, plan = _case(name)
    a = [oeq.oeq_tp_conv_fwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"]) for _ in range(3)]
    b = [oeq.oeq_tp_conv_bwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], mode="deterministic")
         for _ in range(3)]
    c = oeq.oeq_tp_conv_bwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], mode="atomic")
    torch.cuda.synchronize()
    assert all(torch.equal(a[0], t) for t in a[1:])
    for k in range(3):
        assert all(torch.equal(b[0][k], t[k]) for t in b[1:])
    assert torch.equal(b[0][1], c[1]) and torch.equal(b[0][2], c[2])   # gY, gW do not depend on the mode
    assert rel_l2(c[0].cpu().numpy(), b[0][0].cpu().numpy()) <= RTOL[wl.dtype]


# ---------------------------------------------------------------------------
# Full-size workloads, sampled comparison, benchmark launch shape
# ---------------------------------------------------------------------------

def _sampled_fwd_ref(d, inp, rows):
    rp, sr, _ = subgraph(inp["rowptr"], inp["src"], edges_of_rows(inp["rowptr"], rows))
    e = edges_of_rows(inp["rowptr"], rows)
    return oracle.fwd(d, rp, sr, inp["x"], inp["Y"][e], inp["W"][e], rows=rows)


def _sampled_edges_ref(d, inp, edges, x):
    rp, sr, e = subgraph(inp["rowptr"], inp["src"], edges)
    return oracle.bwd_edges(d, rp, sr, x, inp["Y"][e], inp["W"][e], inp["g"])


def _sampled_gx_ref(d, inp, senders, Y, W):
    e = np.nonzero(np.isin(inp["src"], senders))[0]
    rp, sr, e = subgraph(inp["rowptr"], inp["src"], e)
    return oracle.bwd_gx(d, rp, sr, Y[e], W[e], inp["g"], senders=senders)


def _rel_l2_dev(got, ref, rows=1 << 14) -> float:
    """rel_l2 of a device tensor against a host array, over row chunks (no whole
    fp64 copy of a multi-GB output)."""
    num = den = 0.0
    for a in range(0, ref.shape[0], rows):
        g = got[a:a + rows].cpu().numpy().astype(np.float64)
        r = np.asarray(ref[a:a + rows], dtype=np.float64)
        num += float(np.sum((g - r) ** 2))
        den += float(np.sum(r * r))
    return (num ** 0.5) / (den ** 0.5) if den > 0 else (0.0 if num == 0 else float("inf"))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mace_medium_fp32", "mace_medium_fp64", "mace_large_fp32", "invariant_fp32",
                                  "uvw_bcast_medium_fp32", "uvw_sum_medium_fp32"])
def test_full_size_whole(name):
    """The full 5,000-node / 280,000-edge workloads in the benchmark's launch shape,
    compared on every element of every output: forward, VJP in both modes and (for
    the large workload) the HVP.  The two reducible-UVW workloads (a broadcast x block;
    outputs summed over the channels) at the same sizes."""
    wl = synth.by_name(name)
    want = ("x", "Y", "W", "g", "v") if "hvp" in wl.ops else ("x", "Y", "W", "g")
    d, inp = inputs(wl, want=want)
    print(f"[whole] {name} N={wl.n_nodes} E={inp['E']} inputs ready", flush=True)
    g = _dev_inputs(inp, wl.dtype)
    plan = plan_for(wl)
    tol = RTOL[wl.dtype]
    rp, sr = inp["rowptr"], inp["src"]

    out = oeq.oeq_tp_conv_fwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"])
    ref = oracle.fwd(d, rp, sr, inp["x"], inp["Y"], inp["W"])
    assert _rel_l2_dev(out, ref) <= tol
    del out, ref
    print(f"[whole] {name} fwd ok", flush=True)

    rW, rY = oracle.bwd_edges(d, rp, sr, inp["x"], inp["Y"], inp["W"], inp["g"])
    rx = oracle.bwd_gx(d, rp, sr, inp["Y"], inp["W"], inp["g"])
    for mode in ("atomic", "deterministic"):
        gx, gY, gW = oeq.oeq_tp_conv_bwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], mode=mode)
        assert _rel_l2_dev(gx, rx) <= tol
        assert _rel_l2_dev(gY, rY) <= tol
        assert _rel_l2_dev(gW, rW) <= tol
        del gx, gY, gW
        print(f"[whole] {name} bwd {mode} ok", flush=True)
    del rW, rY, rx

    if "hvp" in wl.ops:
        res = oeq.oeq_tp_conv_dbwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], gg_x=g["v"])
        assert not res["x"].any().item()
        ref = oracle.dbwd(d, rp, sr, inp["x"], inp["Y"], inp["W"], inp["g"], ggx=inp["v"], want=("dY", "dW", "dg"))
        assert _rel_l2_dev(res["Y"], ref["dY"]) <= tol
        assert _rel_l2_dev(res["W"], ref["dW"]) <= tol
        assert _rel_l2_dev(res["grad_out"], ref["dg"]) <= tol
        print(f"[whole] {name} hvp ok", flush=True)
    torch.cuda.synchronize()


@pytest.mark.slow
@pytest.mark.parametrize("name", ["wide_proxy_fp32"])
def test_full_size_sampled(name):
    """The wide proxy (6.9 GB of W) at full size, compared on sampled rows: receivers
    for the forward, edges for the W and Y gradients, senders for the x gradient, each
    evaluated by the oracle on the sub-graph of exactly the edges it depends on."""
    wl = W_[name]
    want = ("x", "Y", "W", "g", "v") if "hvp" in wl.ops else ("x", "Y", "W", "g")
    d, inp = inputs(wl, want=want)
    print(f"[full] {name} N={wl.n_nodes} E={inp['E']} inputs ready", flush=True)
    g = _dev_inputs(inp, wl.dtype)
    plan = plan_for(wl)
    tol = RTOL[wl.dtype]
    rows = sample(wl.n_nodes, 40, 1)
    edges = sample(inp["E"], 200, 2)
    senders = sample(wl.n_nodes, 24, 3)
    rows_t, edges_t, send_t = (torch.from_numpy(a).cuda() for a in (rows, edges, senders))

    out = oeq.oeq_tp_conv_fwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"])
    got = out[rows_t].cpu().numpy()
    del out
    assert rel_l2(got, _sampled_fwd_ref(d, inp, rows)) <= tol
    print(f"[full] {name} fwd ok", flush=True)

    rW, rY = _sampled_edges_ref(d, inp, edges, inp["x"])
    rx = _sampled_gx_ref(d, inp, senders, inp["Y"], inp["W"])
    for mode in ("atomic", "deterministic"):
        gx, gY, gW = oeq.oeq_tp_conv_bwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], mode=mode)
        assert rel_l2(gx[send_t].cpu().numpy(), rx) <= tol
        assert rel_l2(gY[edges_t].cpu().numpy(), rY) <= tol
        assert rel_l2(gW[edges_t].cpu().numpy(), rW) <= tol
        del gx, gY, gW
        print(f"[full] {name} bwd {mode} ok", flush=True)

    if "hvp" in wl.ops:
        res = oeq.oeq_tp_conv_dbwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], gg_x=g["v"],
                                   want=("Y", "W", "grad_out"))
        dW, dY = _sampled_edges_ref(d, inp, edges, inp["v"])
        dg = _sampled_fwd_ref(d, dict(inp, x=inp["v"]), rows)
        assert rel_l2(res["Y"][edges_t].cpu().numpy(), dY) <= tol
        assert rel_l2(res["W"][edges_t].cpu().numpy(), dW) <= tol
        assert rel_l2(res["grad_out"][rows_t].cpu().numpy(), dg) <= tol
        print(f"[full] {name} hvp ok", flush=True)
    torch.cuda.synchronize()


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
def test_full_size_double_backward_all_tangents(mode):
    """Double backward with tangents on x, Y and W at full size (the force-training
    path), compared on sampled rows with the oracle's double backward evaluated on
    the sub-graph of exactly the edges each sampled output depends on."""
    wl = W_["mace_large_fp32"]
    d, inp = inputs(wl, want=("x", "Y", "W", "g", "v"))
    tY = synth.extra_normal(wl, inp["Y"].shape, 1)
    tW = synth.extra_normal(wl, inp["W"].shape, 2)
    print(f"[full-dbwd] {mode} inputs ready", flush=True)
    g = _dev_inputs(inp, wl.dtype)
    gY_, gW_ = to_dev(tY), to_dev(tW)
    plan = plan_for(wl)
    res = oeq.oeq_tp_conv_dbwd(plan, g["rowptr"], g["src"], g["x"], g["Y"], g["W"], g["g"], gg_x=g["v"],
                               gg_Y=gY_, gg_W=gW_, mode=mode)
    torch.cuda.synchronize()
    tol = RTOL[wl.dtype]
    rows = sample(wl.n_nodes, 24, 11)
    edges = sample(inp["E"], 160, 12)
    senders = sample(wl.n_nodes, 16, 13)

    def sub(edge_ids):
        rp, sr, e = subgraph(inp["rowptr"], inp["src"], edge_ids)
        return rp, sr, e

    rp, sr, e = sub(edges_of_rows(inp["rowptr"], rows))
    ref = oracle.dbwd(d, rp, sr, inp["x"], inp["Y"][e], inp["W"][e], inp["g"], ggx=inp["v"], ggY=tY[e],
                      ggW=tW[e], rows=rows, want=("dg",))
    assert rel_l2(res["grad_out"][torch.from_numpy(rows).cuda()].cpu().numpy(), ref["dg"]) <= tol
    rp, sr, e = sub(edges)
    ref = oracle.dbwd(d, rp, sr, inp["x"], inp["Y"][e], inp["W"][e], inp["g"], ggx=inp["v"], ggY=tY[e],
                      ggW=tW[e], want=("dY", "dW"))
    et = torch.from_numpy(e).cuda()
    assert rel_l2(res["Y"][et].cpu().numpy(), ref["dY"]) <= tol
    assert rel_l2(res["W"][et].cpu().numpy(), ref["dW"]) <= tol
    rp, sr, e = sub(np.nonzero(np.isin(inp["src"], senders))[0])
    ref = oracle.dbwd(d, rp, sr, inp["x"], inp["Y"][e], inp["W"][e], inp["g"], ggx=inp["v"], ggY=tY[e],
                      ggW=tW[e], senders=senders, want=("dx",))
    assert rel_l2(res["x"][torch.from_numpy(senders).cuda()].cpu().numpy(), ref["dx"]) <= tol
    print(f"[full-dbwd] {mode} ok", flush=True)
