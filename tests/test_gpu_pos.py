"""GPU parity of the convolution driven by atom positions against the oracle
(oracle/positions.py): the forward with the harmonics of pos[s] - pos[r]
evaluated in the kernel, and the VJP returning the gradient to the positions,
scattered to both atoms of every edge by atomics or in a fixed order
(deterministic mode, bitwise repeatable).  The multigraph case has self-loops
(zero edge vectors) and repeated edges.  Bounds as for the other parity tests."""
import numpy as np
import pytest

import oracle
import synth
from helpers import RTOL, oracle_desc, plan_for, rel_l2, sample, to_dev
from oracle import positions
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")

NAMES = ["tiny_fp64", "mace_medium_fp32", "mace_medium_fp64", "mace_large_fp32", "u1_l3_f64", "u8_l1_f32",
         "ragged_u96_f32", "multi_u64_f32", "multi_u40_f64", "ysub_u16_f64"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _case(wl):
    d = oracle_desc(wl)
    inp = synth.generate(wl, d.P, d.out_dim, want=("x", "pos", "W", "g"))
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "pos", "W", "g")}
    return d, inp, dev, plan_for(wl)


@pytest.mark.parametrize("name", NAMES)
def test_fwd_pos_parity(name):
    wl = SMALL[name]
    d, inp, dev, plan = _case(wl)
    print(f"[fwd pos] {name}", flush=True)
    out = oeq.oeq_tp_conv_fwd_pos(plan, dev["rowptr"], dev["src"], dev["x"], dev["pos"], dev["W"])
    torch.cuda.synchronize()
    ref = positions.fwd_pos(d, inp["rowptr"], inp["src"], inp["x"], inp["pos"], inp["W"])
    assert rel_l2(out.cpu().numpy(), ref) <= RTOL[wl.dtype]


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("name", NAMES)
def test_bwd_pos_parity(name, mode):
    wl = SMALL[name]
    d, inp, dev, plan = _case(wl)
    print(f"[bwd pos] {name} {mode}", flush=True)
    args = (dev["rowptr"], dev["src"], dev["x"], dev["pos"], dev["W"], dev["g"])
    gx, gpos, gW = oeq.oeq_tp_conv_bwd_pos(plan, *args, mode=mode)
    again = oeq.oeq_tp_conv_bwd_pos(plan, *args, mode=mode)[1]
    alone = oeq.oeq_tp_conv_bwd_pos(plan, *args, mode=mode, want=("pos",))[1]
    torch.cuda.synchronize()
    rx, rpos, rW = positions.bwd_pos(d, inp["rowptr"], inp["src"], inp["x"], inp["pos"], inp["W"], inp["g"])
    tol = RTOL[wl.dtype]
    assert rel_l2(gx.cpu().numpy(), rx) <= tol
    assert rel_l2(gW.cpu().numpy(), rW) <= tol
    got = gpos.cpu().numpy()
    assert rel_l2(got, rpos) <= tol
    # translation invariance: the gradients sum to zero up to rounding
    assert np.abs(got.astype(np.float64).sum(axis=0)).max() <= 1e3 * np.finfo(got.dtype).eps * np.abs(got).sum()
    if mode == "deterministic":
        assert torch.equal(gpos, again)                       # bitwise repeatable
    assert rel_l2(alone.cpu().numpy(), rpos) <= tol           # the position gradient requested alone


def test_pos_empty_graph():
    wl = synth.WORKLOADS["mace_medium_fp32"].scaled(n_nodes=10, degree=0)
    d, inp, dev, plan = _case(wl)
    out = oeq.oeq_tp_conv_fwd_pos(plan, dev["rowptr"], dev["src"], dev["x"], dev["pos"], dev["W"])
    gx, gpos, gW = oeq.oeq_tp_conv_bwd_pos(plan, dev["rowptr"], dev["src"], dev["x"], dev["pos"], dev["W"], dev["g"],
                                           mode="deterministic")
    torch.cuda.synchronize()
    assert not out.any().item() and not gx.any().item() and not gpos.any().item() and gW.shape[0] == 0


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
def test_pos_full_size_sampled(mode):
    """mace_medium_fp32 at full size from positions: the forward on sampled receivers and
    the position gradient on sampled nodes, each against the oracle on the sub-graph of the
    edges it depends on (a node's gradient depends on its out-edges and its own row)."""
    wl = synth.WORKLOADS["mace_medium_fp32"]
    d, inp, dev, plan = _case(wl)
    print(f"[pos full] {mode} inputs ready", flush=True)
    out = oeq.oeq_tp_conv_fwd_pos(plan, dev["rowptr"], dev["src"], dev["x"], dev["pos"], dev["W"])
    gx, gpos, gW = oeq.oeq_tp_conv_bwd_pos(plan, dev["rowptr"], dev["src"], dev["x"], dev["pos"], dev["W"],
                                           dev["g"], mode=mode)
    torch.cuda.synchronize()
    tol = RTOL[wl.dtype]
    rows = sample(wl.n_nodes, 16, 21)
    rp, sr, e = synth.subgraph(inp["rowptr"], inp["src"], synth.edges_of_rows(inp["rowptr"], rows))
    ref = positions.fwd_pos(d, rp, sr, inp["x"], inp["pos"], inp["W"][e])[rows]
    assert rel_l2(out[torch.from_numpy(rows).cuda()].cpu().numpy(), ref) <= tol
    nodes = sample(wl.n_nodes, 12, 22)
    recv = positions.receivers(inp["rowptr"])
    e = np.nonzero(np.isin(inp["src"], nodes) | np.isin(recv, nodes))[0]
    rp, sr, e = synth.subgraph(inp["rowptr"], inp["src"], e)
    _, rpos, _ = positions.bwd_pos(d, rp, sr, inp["x"], inp["pos"], inp["W"][e], inp["g"])
    assert rel_l2(gpos[torch.from_numpy(nodes).cuda()].cpu().numpy(), rpos[nodes]) <= tol
    print(f"[pos full] {mode} ok", flush=True)
