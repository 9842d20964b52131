"""GPU parity of the kernel variants the planner can choose: path-group counts
for the forward and backward passes, the x-gradient atomic layout, plain
(temporal) weight accesses and the two forms of the forward (CG literals, or
Y-contracted rows in LDS, with several tile sizes).  Each variant is a separate plan (the choice is made
when the plan is compiled) and is compared with the oracle like the defaults."""
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import RTOL, inputs, rel_l2, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _plan(wl, env):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        return oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


CASES = [
    ("mace_large_fp32", {"OEQ_FWD_GROUPS": "1", "OEQ_BWD_GROUPS": "1"}),
    ("mace_large_fp32", {"OEQ_FWD_GROUPS": "4", "OEQ_BWD_GROUPS": "2"}),
    ("mace_large_fp32", {"OEQ_NO_XT": "1", "OEQ_NO_NT": "1"}),
    ("mace_large_fp32", {"OEQ_FWD_GROUPS": "3", "OEQ_PIN": "fb", "OEQ_FWD_WAVES": "1,2"}),
    ("mace_medium_fp64", {"OEQ_FWD_GROUPS": "3", "OEQ_BWD_GROUPS": "1", "OEQ_GY_TILE": "7"}),
    ("tiny_fp64", {"OEQ_FWD_GROUPS": "6", "OEQ_BWD_GROUPS": "2"}),
    ("tiny_fp64", {"OEQ_DBWD_SPLIT": "1", "OEQ_BWD_GROUPS": "2"}),
    ("tiny_fp64", {"OEQ_DBWD_SPLIT": "2", "OEQ_BWD_GROUPS": "2"}),
    ("mace_medium_fp32", {"OEQ_DBWD_SPLIT": "1"}),
    ("mace_medium_fp32", {"OEQ_DBWD_SPLIT": "2"}),
    ("mace_medium_fp32", {"OEQ_DBWD_SPLIT": "0"}),
    # double-backward path groups other than the planned ones, with each split level
    ("mace_medium_fp32", {"OEQ_DBWD_GROUPS": "2"}),
    ("mace_large_fp32", {"OEQ_DBWD_GROUPS": "1"}),
    ("mace_large_fp32", {"OEQ_DBWD_GROUPS": "2", "OEQ_DBWD_SPLIT": "1"}),
    ("mace_medium_fp64", {"OEQ_DBWD_GROUPS": "2", "OEQ_DBWD_SPLIT": "2"}),
    # forward from Y-contracted CG rows in LDS (the default for fp64 and for four or more
    # channel chunks) and the literal form: tiles of one edge, of 7 (ragged), 32, 50 and 64
    ("mace_medium_fp64", {"OEQ_FWD_LDS": "0"}),
    ("tiny_fp64", {"OEQ_FWD_LDS": "0"}),
    ("mace_medium_fp32", {"OEQ_FWD_LDS": "1"}),
    ("mace_medium_fp32", {"OEQ_FWD_LDS": "1", "OEQ_FWD_TILE": "32"}),
    ("wide_proxy_fp32", {"OEQ_FWD_LDS": "0"}),
    ("mace_medium_fp32", {"OEQ_FWD_LDS": "1", "OEQ_FWD_TILE": "1"}),
    ("mace_large_fp32", {"OEQ_FWD_LDS": "1", "OEQ_FWD_TILE": "7", "OEQ_FWD_GROUPS": "3"}),
    ("wide_proxy_fp32", {"OEQ_FWD_LDS": "1", "OEQ_FWD_TILE": "100"}),
    # forward workgroups of one channel chunk in an XCD-affine order, both forms
    ("mace_medium_fp32", {"OEQ_FWD_XCD": "1"}),
    ("wide_proxy_fp32", {"OEQ_FWD_XCD": "1", "OEQ_FWD_LDS": "1"}),
    ("mace_medium_fp64", {"OEQ_FWD_XCD": "1"}),
    # loads one edge ahead in the forward (the default is two), two edges ahead in the VJP
    ("mace_medium_fp32", {"OEQ_FWD_PF": "1"}),
    ("mace_large_fp32", {"OEQ_FWD_PF": "1", "OEQ_BWD_PF": "2"}),
    ("tiny_fp64", {"OEQ_FWD_LDS": "0", "OEQ_BWD_PF": "2"}),
    # the HVP from Y-contracted CG rows in LDS (an option): one backward group, and two
    # groups (partial Y-gradient rows) with ragged tiles of 7 edges
    ("mace_medium_fp32", {"OEQ_HVP_LDS": "1"}),
    ("tiny_fp64", {"OEQ_HVP_LDS": "1", "OEQ_BWD_GROUPS": "2", "OEQ_HVP_TILE": "7"}),
    # the split double backward's accumulating forward launches in the tile form
    ("mace_medium_fp64", {"OEQ_DBWD_SPLIT": "1"}),
    ("mace_medium_fp32", {"OEQ_FWD_LDS": "1", "OEQ_DBWD_SPLIT": "2"}),
]


@pytest.mark.parametrize("name,env", CASES, ids=[f"{n}-{'-'.join(f'{k[4:]}{v}' for k, v in e.items())}"
                                                 for n, e in CASES])
def test_variant_parity(name, env):
    wl = synth.WORKLOADS[name]
    if wl.n_nodes > 200:
        wl = wl.scaled(n_nodes=120)
    d, inp = inputs(wl, want=("x", "Y", "W", "g", "v"))
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "W", "g", "v")}
    plan = _plan(wl, env)
    print(f"[variant] {name} {env}", flush=True)
    tol = RTOL[wl.dtype]
    out = oeq.oeq_tp_conv_fwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"])
    ref = oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"])
    assert rel_l2(out.cpu().numpy(), ref) <= tol
    rx, rY, rW = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"])
    for mode in ("atomic", "deterministic"):
        gx, gY, gW = oeq.oeq_tp_conv_bwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                                         mode=mode)
        assert rel_l2(gx.cpu().numpy(), rx) <= tol
        assert rel_l2(gY.cpu().numpy(), rY) <= tol
        assert rel_l2(gW.cpu().numpy(), rW) <= tol
    tY = synth.extra_normal(wl, inp["Y"].shape, 1)
    tYd = to_dev(tY)
    # every tangent set, all outputs and each output alone; outputs start as NaN so
    # a pass that leaves one unwritten fails
    shapes = {"x": inp["x"].shape, "Y": inp["Y"].shape, "W": inp["W"].shape, "grad_out": inp["g"].shape}
    for mask in range(1, 8):
        refd = oracle.dbwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"],
                           ggx=inp["v"] if mask & 1 else None, ggY=tY if mask & 2 else None,
                           ggW=inp["W"] if mask & 4 else None)
        for mode in ("atomic", "deterministic"):
            for want in (("x", "Y", "W", "grad_out"), ("x",), ("Y",), ("W",), ("grad_out",)):
                if len(want) == 1 and mask not in (3, 7):
                    continue
                res = {k: torch.full(shapes[k], float("nan"), dtype=plan.torch_dtype(), device="cuda")
                       for k in want}
                oeq.oeq_tp_conv_dbwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                                     gg_x=dev["v"] if mask & 1 else None, gg_Y=tYd if mask & 2 else None,
                                     gg_W=dev["W"] if mask & 4 else None, mode=mode, out=res)
                for k, rk in (("x", "dx"), ("Y", "dY"), ("W", "dW"), ("grad_out", "dg")):
                    if k not in want:
                        continue
                    got = res[k].cpu().numpy()
                    if not np.any(refd[rk]):
                        assert not got.any(), (mask, mode, want, k)
                    else:
                        assert rel_l2(got, refd[rk]) <= tol, (mask, mode, want, k)
    torch.cuda.synchronize()
