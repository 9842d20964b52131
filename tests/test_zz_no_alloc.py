"""The allocation-free backward entry point, oeq_tp_conv_bwd_noalloc, against
oeq_tp_conv_bwd on the same inputs, through the C ABI.

Two calls in a row on one device, the second on a smaller graph (the shared
device scratch keeps the first call's contents), in both x-gradient modes: the
deterministic mode keeps its per-edge rows and sender CSR in the scratch and must
match bit for bit; the atomic mode within the fp tolerance.  A plan whose backward
runs in two path groups puts its partial Y-gradient rows there too, and a plan with a
one-channel x block its atomic x-gradient rows of U channels per block.  A plan whose
kernels are not yet loaded on the device is refused (loading allocates)."""
import numpy as np
import pytest

import synth
from helpers import RTOL, inputs, plan_for, rel_l2, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


W_ = synth.WORKLOADS
_UVW = synth.Workload("reducible_uvw", 150, 24, synth._irr("1x0e+96x1o+96x2e"), 2, 2, "f32", "unit", 67,
                      out_irreps=synth._irr("96x0e+1x1o+96x1e+96x2e+1x2o"))
CASES = {
    # (larger graph, smaller graph, planner options)
    "medium_fp32": (W_["mace_medium_fp32"].scaled(n_nodes=240), W_["mace_medium_fp32"].scaled(n_nodes=90, seed=7),
                    {}),
    "medium_fp64": (W_["mace_medium_fp64"].scaled(n_nodes=120), W_["mace_medium_fp64"].scaled(n_nodes=60, seed=8),
                    {}),
    "large_two_groups": (W_["mace_large_fp32"].scaled(n_nodes=160), W_["mace_large_fp32"].scaled(n_nodes=70, seed=9),
                         {"OEQ_BWD_GROUPS": "2"}),
    # a broadcast x block and channel sums: the atomic mode's x-gradient rows of U channels
    # per block are in the scratch too
    "reducible_uvw": (_UVW.scaled(n_nodes=150), _UVW.scaled(n_nodes=50, seed=10), {}),
}


def _pair(plan, wl, mode):
    _, inp = inputs(wl)
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "W", "g")}
    args = (dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"])
    ref = oeq.oeq_tp_conv_bwd(plan, *args, mode=mode)
    got = tuple(torch.full_like(t, float("nan")) for t in ref)
    oeq.oeq_tp_conv_bwd_noalloc(plan, *args, out=got, mode=mode)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("mode", ["deterministic", "atomic"])
@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_bwd_on_two_calls(name, mode):
    big, small, env = CASES[name]
    plan = plan_for(big, env)
    for wl in (big, small):
        print(f"[noalloc] {name} {mode} N={wl.n_nodes}", flush=True)
        ref, got = _pair(plan, wl, mode)
        for k, a, b in zip(("x", "Y", "W"), ref, got):
            if mode == "deterministic":
                assert torch.equal(a, b), k
            else:
                assert rel_l2(b.cpu().numpy(), a.cpu().numpy()) <= RTOL[wl.dtype], k


def test_noalloc_refuses_a_plan_not_loaded_on_the_device():
    wl = W_["tiny_fp64"]
    _, inp = inputs(wl)
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "W", "g")}
    args = (dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"])
    plan = plan_for(wl)                                   # a new plan: no kernels loaded yet
    out = tuple(torch.empty_like(t) for t in (dev["x"], dev["Y"], dev["W"]))
    with pytest.raises(oeq.OeqError) as e:
        oeq.oeq_tp_conv_bwd_noalloc(plan, *args, out=out, mode="deterministic")
    assert e.value.status == 1
    ref = oeq.oeq_tp_conv_bwd(plan, *args, mode="deterministic")
    oeq.oeq_tp_conv_bwd_noalloc(plan, *args, out=out, mode="deterministic")
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(ref, out))
