"""GPU parity of the UVW products that reduce to the channel-wise one, against the
oracle: x blocks of one channel broadcast against the U channels, and output
blocks of one channel that receive the sum over the channels.  Forward in both
of its forms, VJP in both modes, the HVP and every double-backward tangent mix,
and the forward and VJP from edge vectors and from positions.  Bounds as for the
other parity tests (relative L2 1e-5 fp32, 1e-12 fp64)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import RTOL, inputs, plan_for, rel_l2, to_dev
from oracle import positions

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")

_I = synth._irr
_deg = np.random.default_rng(81).integers(0, 61, size=90)
_deg[[0, 44, 89]] = 0
CASES = {
    # a broadcast scalar beside 64 vector channels; every output block keeps U channels
    "bcast_u64_f32": synth.Workload("bcast_u64_f32", 120, 20, _I("1x0e+64x1o"), 2, 3, "f32", "unit", 61),
    # channel sums into three of five output blocks
    "sum_u64_f32": synth.Workload("sum_u64_f32", 100, 24, _I("64x0e+64x1o"), 2, 2, "f32", "unit", 62,
                                  out_irreps=_I("1x0e+64x1o+1x1e+64x2e+1x2o")),
    # both readings, U = 96 (a full wave and a half-empty one), ragged degrees with empty rows
    "mixed_u96_f64": synth.Workload("mixed_u96_f64", 90, 0, _I("1x0e+96x1o+1x2e"), 2, 2, "f64", "unit", 63,
                                    degrees=tuple(int(v) for v in _deg),
                                    out_irreps=_I("1x0e+96x1o+96x0o+1x1e+96x2e+1x2o")),
    # four channel chunks (the forward's Y-contracted rows in LDS by default)
    "sum_u256_f32": synth.Workload("sum_u256_f32", 48, 30, _I("256x0e+256x1o"), 3, 3, "f32", "unit", 64,
                                   out_irreps=_I("1x0e+256x1o+1x1e+256x2e+1x2o+256x3o+1x3e")),
    # a multigraph (self-loops, repeated edges) with a partial wave (U = 40), both readings
    "mixed_u40_multi_f32": synth.Workload("mixed_u40_multi_f32", 60, 0, _I("40x0e+1x1o+40x1e"), 2, 2, "f32",
                                          "unit", 65, degrees=tuple(int(v) for v in _deg[:60]), multi=True,
                                          out_irreps=_I("40x0e+1x1o+1x1e+40x2e+1x0o")),
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _case(name, env=None, want=("x", "Y", "W", "g", "v")):
    wl = CASES[name]
    d, inp = inputs(wl, want=want)
    dev = {k: to_dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    return wl, d, inp, dev, plan_for(wl, env)


def _paths_match(plan, d):
    got = [(p[0], p[2], p[3], p[4]) for p in plan.paths()]
    want = [(i1, d.path_l2(k), l3, ob) for k, (i1, _j, l3, ob) in enumerate(d.paths)]
    assert got == want
    assert (plan.x_dim, plan.out_dim, plan.U) == (d.x_dim, d.out_dim, d.U)


def _tile_form(wl):
    return wl.dtype == "f64" or wl.U > 192


@pytest.mark.parametrize("form", ["default", "other"])
@pytest.mark.parametrize("name", list(CASES))
def test_fwd_parity(name, form):
    wl = CASES[name]
    env = None if form == "default" else {"OEQ_FWD_LDS": "0" if _tile_form(wl) else "1"}
    wl, d, inp, dev, plan = _case(name, env)
    _paths_match(plan, d)
    print(f"[uvw fwd] {name} {form} N={wl.n_nodes} E={inp['E']}", flush=True)
    out = oeq.oeq_tp_conv_fwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"])
    torch.cuda.synchronize()
    ref = oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"])
    assert rel_l2(out.cpu().numpy(), ref) <= RTOL[wl.dtype]
    deg = np.diff(inp["rowptr"])
    assert not out.cpu().numpy()[deg == 0].any()


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("name", list(CASES))
def test_bwd_parity(name, mode):
    wl, d, inp, dev, plan = _case(name)
    print(f"[uvw bwd] {name} {mode}", flush=True)
    gx, gY, gW = oeq.oeq_tp_conv_bwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                                     mode=mode)
    torch.cuda.synchronize()
    rx, rY, rW = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"])
    tol = RTOL[wl.dtype]
    assert rel_l2(gx.cpu().numpy(), rx) <= tol
    assert rel_l2(gY.cpu().numpy(), rY) <= tol
    assert rel_l2(gW.cpu().numpy(), rW) <= tol


@pytest.mark.parametrize("name", list(CASES))
def test_bwd_deterministic_is_bitwise_repeatable(name):
    wl, d, inp, dev, plan = _case(name)
    args = (plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"])
    a = oeq.oeq_tp_conv_bwd(*args, mode="deterministic")
    b = oeq.oeq_tp_conv_bwd(*args, mode="deterministic")
    f1 = oeq.oeq_tp_conv_fwd(*args[:6])
    f2 = oeq.oeq_tp_conv_fwd(*args[:6])
    torch.cuda.synchronize()
    for u, v in zip(a + (f1,), b + (f2,)):
        assert torch.equal(u, v)


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("mask", [1, 2, 4, 7])
@pytest.mark.parametrize("name", ["bcast_u64_f32", "sum_u64_f32", "mixed_u96_f64", "mixed_u40_multi_f32"])
def test_dbwd_parity(name, mask, mode):
    wl, d, inp, dev, plan = _case(name)
    tx = synth.extra_normal(wl, inp["x"].shape, 0)
    tY = synth.extra_normal(wl, inp["Y"].shape, 1)
    tW = synth.extra_normal(wl, inp["W"].shape, 2)
    print(f"[uvw dbwd] {name} {mask} {mode}", flush=True)
    res = oeq.oeq_tp_conv_dbwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                               gg_x=to_dev(tx) if mask & 1 else None, gg_Y=to_dev(tY) if mask & 2 else None,
                               gg_W=to_dev(tW) if mask & 4 else None, mode=mode)
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


@pytest.mark.parametrize("name", ["bcast_u64_f32", "mixed_u96_f64", "sum_u256_f32"])
def test_vec_and_pos_parity(name):
    wl, d, inp, dev, plan = _case(name, want=("x", "vec", "pos", "W", "g"))
    print(f"[uvw vec/pos] {name}", flush=True)
    tol = RTOL[wl.dtype]
    vec = inp["vec"].astype(wl.np_dtype())       # the vectors the kernel sees
    dev["vec"] = to_dev(vec)
    Y = synth.real_sh_cartesian(max(wl.y_degrees), vec.astype(np.float64))
    out = oeq.oeq_tp_conv_fwd_vec(plan, dev["rowptr"], dev["src"], dev["x"], dev["vec"], dev["W"])
    gx, gvec, gW = oeq.oeq_tp_conv_bwd_vec(plan, dev["rowptr"], dev["src"], dev["x"], dev["vec"], dev["W"], dev["g"])
    outp = oeq.oeq_tp_conv_fwd_pos(plan, dev["rowptr"], dev["src"], dev["x"], dev["pos"], dev["W"])
    gxp, gpos, gWp = oeq.oeq_tp_conv_bwd_pos(plan, dev["rowptr"], dev["src"], dev["x"], dev["pos"], dev["W"],
                                             dev["g"])
    torch.cuda.synchronize()
    assert rel_l2(out.cpu().numpy(), oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], Y, inp["W"])) <= tol
    rx, _rY, rW = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], Y, inp["W"], inp["g"])
    assert rel_l2(gx.cpu().numpy(), rx) <= tol and rel_l2(gW.cpu().numpy(), rW) <= tol
    ref = positions.fwd_pos(d, inp["rowptr"], inp["src"], inp["x"], inp["pos"], inp["W"])
    assert rel_l2(outp.cpu().numpy(), ref) <= tol
    rxp, rpos, rWp = positions.bwd_pos(d, inp["rowptr"], inp["src"], inp["x"], inp["pos"], inp["W"], inp["g"])
    assert rel_l2(gxp.cpu().numpy(), rxp) <= tol
    assert rel_l2(gpos.cpu().numpy(), rpos) <= tol
    assert rel_l2(gWp.cpu().numpy(), rWp) <= tol


def test_forward_accumulates_into_out_for_the_double_backward():
    """d_grad_out of a plan with channel sums comes from the forward kernel, which adds
    its sums into the row when asked (all three tangents: three accumulating launches)."""
    wl, d, inp, dev, plan = _case("sum_u64_f32")
    tx = synth.extra_normal(wl, inp["x"].shape, 0)
    tY = synth.extra_normal(wl, inp["Y"].shape, 1)
    tW = synth.extra_normal(wl, inp["W"].shape, 2)
    res = oeq.oeq_tp_conv_dbwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                               gg_x=to_dev(tx), gg_Y=to_dev(tY), gg_W=to_dev(tW), want=("grad_out",))
    torch.cuda.synchronize()
    rp, sr = inp["rowptr"], inp["src"]
    ref = (oracle.fwd(d, rp, sr, tx, inp["Y"], inp["W"]) + oracle.fwd(d, rp, sr, inp["x"], tY, inp["W"])
           + oracle.fwd(d, rp, sr, inp["x"], inp["Y"], tW))
    assert rel_l2(res["grad_out"].cpu().numpy(), ref) <= RTOL[wl.dtype]


PATHLESS = {
    # an output irrep that no path reaches (0o: no x block and Y block combine to it), in a
    # plan with U channels everywhere and in one with channel sums
    "pathless_u32_f32": synth.Workload("pathless_u32_f32", 70, 12, _I("32x0e+32x1o"), 1, 2, "f32", "unit", 66,
                                       out_irreps=_I("32x0e+32x1o+32x0o+32x1e")),
    "mixed_u96_f64": CASES["mixed_u96_f64"],
}


@pytest.mark.parametrize("name", list(PATHLESS))
def test_output_blocks_without_paths_are_written_as_zero(name):
    """Every output element is written, also those of a block no path reaches (the sum
    over no paths): outputs start as NaN and must come back equal to the oracle."""
    wl = PATHLESS[name]
    d, inp = inputs(wl, want=("x", "Y", "W", "g", "v"))
    dev = {k: to_dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    plan = plan_for(wl)
    print(f"[uvw pathless] {name}", flush=True)
    nan = torch.full((wl.n_nodes, plan.out_dim), float("nan"), dtype=plan.torch_dtype(), device="cuda")
    out = oeq.oeq_tp_conv_fwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], out=nan.clone())
    dg = {"grad_out": nan.clone()}
    res = oeq.oeq_tp_conv_dbwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                               gg_x=dev["v"], want=("grad_out",), out=dg)
    torch.cuda.synchronize()
    rp, sr = inp["rowptr"], inp["src"]
    ref = oracle.fwd(d, rp, sr, inp["x"], inp["Y"], inp["W"])
    got = out.cpu().numpy()
    assert not np.isnan(got).any() and rel_l2(got, ref) <= RTOL[wl.dtype]
    fed = {ob for (*_, ob) in d.paths}
    o = 0
    for b, (m, l) in enumerate(zip(d.out_mul, d.out_l)):
        if b not in fed:
            assert not got[:, o:o + m * (2 * l + 1)].any()
        o += m * (2 * l + 1)
    refg = oracle.fwd(d, rp, sr, inp["v"], inp["Y"], inp["W"])
    gg = res["grad_out"].cpu().numpy()
    assert not np.isnan(gg).any() and rel_l2(gg, refg) <= RTOL[wl.dtype]


@pytest.mark.parametrize("split", ["0", "1", "2"])
@pytest.mark.parametrize("name", ["sum_u64_f32", "mixed_u96_f64", "sum_u256_f32"])
def test_dbwd_split_levels_with_channel_sums(name, split):
    """The fused double backward sums one-channel d_grad_out blocks in LDS; the split
    passes take d_grad_out from the forward kernel.  Each level against the oracle, with
    outputs that start as NaN."""
    wl, d, inp, dev, plan = _case(name, {"OEQ_DBWD_SPLIT": split})
    tx = synth.extra_normal(wl, inp["x"].shape, 0)
    tY = synth.extra_normal(wl, inp["Y"].shape, 1)
    tW = synth.extra_normal(wl, inp["W"].shape, 2)
    print(f"[uvw dbwd split] {name} {split}", flush=True)
    shapes = {"x": inp["x"].shape, "Y": inp["Y"].shape, "W": inp["W"].shape, "grad_out": inp["g"].shape}
    for mask in (1, 7):
        ref = oracle.dbwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"],
                          ggx=tx, ggY=tY if mask & 2 else None, ggW=tW if mask & 4 else None)
        res = {k: torch.full(v, float("nan"), dtype=plan.torch_dtype(), device="cuda") for k, v in shapes.items()}
        oeq.oeq_tp_conv_dbwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                             gg_x=to_dev(tx), gg_Y=to_dev(tY) if mask & 2 else None,
                             gg_W=to_dev(tW) if mask & 4 else None, out=res)
        torch.cuda.synchronize()
        for k, rk in (("x", "dx"), ("Y", "dY"), ("W", "dW"), ("grad_out", "dg")):
            got = res[k].cpu().numpy()
            if not np.any(ref[rk]):
                assert not got.any(), (mask, k)
            else:
                assert rel_l2(got, ref[rk]) <= RTOL[wl.dtype], (mask, k)
