"""GPU parity of the sender-stationary schedule (the "source stationary" variant
the maintainers propose in "Receiver-streaming convolutions for channel-wise UVU
tensor products", maintainer reply) against the CPU oracle, through the C ABI:
the sender view of the graph (bit-exact), the forward with atomically scattered
messages and the VJP whose x gradient is accumulated per sender without atomics
(bitwise repeatable).  Bounds as in the receiver-stationary parity tests."""
import numpy as np
import pytest

import oracle
import synth
from helpers import RTOL, inputs, plan_for, rel_l2, sample, to_dev
from test_gpu_parity import SMALL, _sampled_edges_ref, _sampled_fwd_ref, _sampled_gx_ref

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")

CASES = SMALL


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _case(name):
    wl = CASES[name]
    d, inp = inputs(wl, want=("x", "Y", "W", "g"))
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "W", "g")}
    return wl, d, inp, dev, plan_for(wl)


def _receivers_in_sender_order(rowptr, sperm):
    """The receiver of each edge sperm[k]: the CSR row that holds it."""
    return (np.searchsorted(rowptr, sperm, side="right") - 1).astype(np.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_sender_view_bit_exact(name):
    wl, d, inp, dev, plan = _case(name)
    print(f"[view] {name}", flush=True)
    srowptr, sperm, sdst = oeq.oeq_sender_view(dev["rowptr"], dev["src"])
    torch.cuda.synchronize()
    ref_rp, ref_perm = oracle.sender_csr(wl.n_nodes, inp["src"])
    assert np.array_equal(srowptr.cpu().numpy(), ref_rp)
    assert np.array_equal(sperm.cpu().numpy(), ref_perm)
    assert np.array_equal(sdst.cpu().numpy(), _receivers_in_sender_order(inp["rowptr"], ref_perm))


@pytest.mark.parametrize("name", list(CASES))
def test_fwd_sender_parity(name):
    wl, d, inp, dev, plan = _case(name)
    print(f"[fwd sender] {name} N={wl.n_nodes} E={inp['E']}", flush=True)
    view = oeq.oeq_sender_view(dev["rowptr"], dev["src"])
    out = torch.full((wl.n_nodes, plan.out_dim), float("nan"), dtype=plan.torch_dtype(), device="cuda")
    oeq.oeq_tp_conv_fwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], out=out)
    torch.cuda.synchronize()
    ref = oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"])
    got = out.cpu().numpy()
    assert rel_l2(got, ref) <= RTOL[wl.dtype]
    assert not got[np.diff(inp["rowptr"]) == 0].any()     # receivers without edges


@pytest.mark.parametrize("name", list(CASES))
def test_bwd_sender_parity_and_repeatable(name):
    wl, d, inp, dev, plan = _case(name)
    print(f"[bwd sender] {name} N={wl.n_nodes} E={inp['E']}", flush=True)
    view = oeq.oeq_sender_view(dev["rowptr"], dev["src"])
    first = oeq.oeq_tp_conv_bwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], dev["g"])
    second = oeq.oeq_tp_conv_bwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], dev["g"])
    torch.cuda.synchronize()
    ref = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"])
    for a, b, r in zip(first, second, ref):
        assert rel_l2(a.cpu().numpy(), r) <= RTOL[wl.dtype]
        assert torch.equal(a, b)                          # no atomics: bitwise repeatable


@pytest.mark.parametrize("name", ["mace_medium_fp32", "u8_l1_f32", "invariant_fp32"])
def test_bwd_sender_partial_outputs(name):
    wl, d, inp, dev, plan = _case(name)
    view = oeq.oeq_sender_view(dev["rowptr"], dev["src"])
    full = oeq.oeq_tp_conv_bwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], dev["g"])
    for want in (("x",), ("Y",), ("W",), ("x", "W")):
        part = oeq.oeq_tp_conv_bwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], dev["g"], want=want)
        for k, a, b in zip(("x", "Y", "W"), full, part):
            if k in want:
                assert torch.equal(a, b), (want, k)
            else:
                assert b is None


def test_sender_unused_x_block_and_shared_output_block():
    """An explicit path list that leaves an x block unused (its gradient must be
    zero) and sums two paths into one output block."""
    x_irreps = ((8, 0, 1), (8, 1, -1), (8, 2, 1))
    paths = [(0, 1, 0), (2, 1, 0)]            # 0e x 1o -> 1o and 2e x 1o -> 1o, both into block 0
    wl = synth.Workload("explicit", 60, 7, x_irreps, 1, 1, "f64", "unit", 41)
    d = oracle.Desc(x_irreps, 1, paths=[(0, 1, 1, 0), (2, 1, 1, 0)], out_l=[1])
    inp = synth.generate(wl, d.P, d.out_dim, want=("x", "Y", "W", "g"))
    plan = oeq.Plan(x_irreps, 1, 1, "f64", paths=paths, out_irreps=((8, 1, -1),))
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "W", "g")}
    view = oeq.oeq_sender_view(dev["rowptr"], dev["src"])
    out = oeq.oeq_tp_conv_fwd_sender(plan, view, dev["x"], dev["Y"], dev["W"])
    gx = torch.full((wl.n_nodes, plan.x_dim), float("nan"), dtype=torch.float64, device="cuda")
    oeq.oeq_tp_conv_bwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], dev["g"], want=("x",),
                               out=(gx, None, None))
    torch.cuda.synchronize()
    assert rel_l2(out.cpu().numpy(), oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"])) <= 1e-12
    rx, _, _ = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"])
    got = gx.cpu().numpy()
    assert rel_l2(got, rx) <= 1e-12
    assert not got[:, 8:32].any()                   # the 1o block feeds no path
    # the receiver-stationary VJP and double backward, deterministic mode (per-edge rows)
    for mode in ("atomic", "deterministic"):
        gxr, _, _ = oeq.oeq_tp_conv_bwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                                        mode=mode)
        got = gxr.cpu().numpy()
        assert rel_l2(got, rx) <= 1e-12 and not got[:, 8:32].any(), mode
        tY = synth.extra_normal(wl, inp["Y"].shape, 2)
        res = oeq.oeq_tp_conv_dbwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                                   gg_Y=to_dev(tY), mode=mode, want=("x",))
        refd = oracle.dbwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"], ggY=tY)
        got = res["x"].cpu().numpy()
        assert rel_l2(got, refd["dx"]) <= 1e-12 and not got[:, 8:32].any(), mode


def test_sender_empty_graph():
    wl = synth.WORKLOADS["tiny_fp64"]
    plan = plan_for(wl)
    N = 5
    rowptr = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    src = torch.zeros(0, dtype=torch.int32, device="cuda")
    view = oeq.oeq_sender_view(rowptr, src)
    x = torch.randn(N, plan.x_dim, dtype=torch.float64, device="cuda")
    Y = torch.zeros(0, plan.y_dim, dtype=torch.float64, device="cuda")
    W = torch.zeros(0, plan.n_paths, plan.U, dtype=torch.float64, device="cuda")
    g = torch.randn(N, plan.out_dim, dtype=torch.float64, device="cuda")
    out = oeq.oeq_tp_conv_fwd_sender(plan, view, x, Y, W)
    gx, gY, gW = oeq.oeq_tp_conv_bwd_sender(plan, view, x, Y, W, g)
    torch.cuda.synchronize()
    assert view[0].cpu().numpy().tolist() == [0] * (N + 1)
    assert not out.cpu().numpy().any() and not gx.cpu().numpy().any()
    assert gY.shape == (0, plan.y_dim) and gW.shape == (0, plan.n_paths, plan.U)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["invariant_fp32", "mace_medium_fp32"])
def test_sender_full_size_sampled(name):
    """Full 5,000-node / 280,000-edge graph in the benchmark's launch shape,
    compared on sampled receivers, edges and senders."""
    wl = synth.WORKLOADS[name]
    d, inp = inputs(wl, want=("x", "Y", "W", "g"))
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "W", "g")}
    plan = plan_for(wl)
    print(f"[sender full] {name}", flush=True)
    view = oeq.oeq_sender_view(dev["rowptr"], dev["src"])
    out = oeq.oeq_tp_conv_fwd_sender(plan, view, dev["x"], dev["Y"], dev["W"])
    gx, gY, gW = oeq.oeq_tp_conv_bwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], dev["g"])
    torch.cuda.synchronize()
    tol = RTOL[wl.dtype]
    rows, edges, senders = sample(wl.n_nodes, 24, 5), sample(inp["E"], 300, 6), sample(wl.n_nodes, 24, 7)
    rows_t, edges_t, send_t = (torch.from_numpy(a).cuda() for a in (rows, edges, senders))
    assert rel_l2(out[rows_t].cpu().numpy(), _sampled_fwd_ref(d, inp, rows)) <= tol
    rW, rY = _sampled_edges_ref(d, inp, edges, inp["x"])
    assert rel_l2(gW[edges_t].cpu().numpy(), rW) <= tol
    assert rel_l2(gY[edges_t].cpu().numpy(), rY) <= tol
    rx = _sampled_gx_ref(d, inp, senders, inp["Y"], inp["W"])
    assert rel_l2(gx[send_t].cpu().numpy(), rx) <= tol


def _schedule_bwd(wl):
    return plan_for(wl).schedule()["bwd"]


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("name", ["invariant_fp32", "u8_l1_f32", "tiny_fp64", "ysub_u16_f64"])
def test_bwd_follows_the_plans_schedule(name, mode):
    """oeq_tp_conv_bwd runs the pass the plan's data-movement model prefers: on these plans
    the sender-stationary one, whose results (built on a sender view it makes in the
    workspace) equal the explicit sender-stationary call bit for bit in either mode.  A
    plan forced to the receiver-stationary VJP (OEQ_SCHEDULE=rr) agrees within tolerance."""
    wl, d, inp, dev, plan = _case(name)
    assert plan.schedule()["bwd"] == "sender"
    args = (dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"])
    auto = oeq.oeq_tp_conv_bwd(plan, *args, mode=mode)
    view = oeq.oeq_sender_view(dev["rowptr"], dev["src"])
    explicit = oeq.oeq_tp_conv_bwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], dev["g"])
    forced = oeq.oeq_tp_conv_bwd(plan_for(wl, {"OEQ_SCHEDULE": "rr"}), *args, mode=mode)
    torch.cuda.synchronize()
    ref = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"])
    for a, b, c, r in zip(auto, explicit, forced, ref):
        assert torch.equal(a, b)
        assert rel_l2(a.cpu().numpy(), r) <= RTOL[wl.dtype]
        assert rel_l2(c.cpu().numpy(), r) <= RTOL[wl.dtype]
