"""GPU parity of the radial-weight passes (sine basis with a polynomial cutoff,
one SiLU hidden layer, linear output; dense products on the matrix cores)
against the oracle (oracle/radial.py): the weights, and the gradients to the
edge vectors and to both weight matrices, including hidden widths that are not
multiples of the 16-wide matrix blocks, lengths beyond the cutoff and a zero
vector."""
import os

import numpy as np
import pytest

import synth
from helpers import RTOL, plan_for, rel_l2, sample, to_dev
from oracle import radial
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")

RC = 6.0


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _problem(wl, plan, H, seed, E=None):
    rng = np.random.default_rng(seed)
    d = synth.generate(wl, plan.n_paths, plan.out_dim, want=("evec",))
    vec = d["evec"] if E is None else d["evec"][:E]
    # beyond the cutoff, on it, and a zero vector
    extra = np.array([[7.0, 0, 0], [0, -RC, 0], [0, 0, 0], [0.3, 0.2, -0.1]], dtype=wl.np_dtype())
    vec = np.concatenate([vec, extra])
    PU = plan.n_paths * plan.U
    dt = wl.np_dtype()
    W1 = rng.standard_normal((8, H)).astype(dt)
    W2 = rng.standard_normal((H, PU)).astype(dt)
    gW = rng.standard_normal((len(vec), PU)).astype(dt)
    return vec, W1, W2, gW


CASES = [("tiny_fp64", 16), ("tiny_fp64", 40), ("mace_medium_fp32", 64), ("mace_medium_fp64", 64),
         ("mace_large_fp32", 24), ("u1_l3_f64", 64), ("ragged_u96_f32", 72), ("u8_l1_f32", 8)]


@pytest.mark.parametrize("name,H", CASES)
def test_radial_parity(name, H):
    wl = SMALL[name]
    plan = plan_for(wl)
    vec, W1, W2, gW = _problem(wl, plan, H, 5, E=3000)
    print(f"[radial] {name} H={H} E={len(vec)}", flush=True)
    dv, d1, d2, dg = (to_dev(a) for a in (vec, W1, W2, gW.reshape(len(vec), plan.n_paths, plan.U)))
    W = oeq.oeq_radial_fwd(plan, dv, RC, d1, d2)
    g = oeq.oeq_radial_bwd(plan, dv, RC, d1, d2, dg)
    g_again = oeq.oeq_radial_bwd(plan, dv, RC, d1, d2, dg)
    torch.cuda.synchronize()
    tol = RTOL[wl.dtype]
    refW = radial.radial_fwd(vec, RC, W1, W2)
    assert rel_l2(W.cpu().numpy().reshape(len(vec), -1), refW) <= tol
    assert not W[-4:-2].cpu().numpy().any()           # beyond and on the cutoff: zero weights
    rv, r1, r2 = radial.radial_bwd(vec, RC, W1, W2, gW)
    for got, ref, k in zip(g, (rv, r1, r2), ("vec", "W1", "W2")):
        assert rel_l2(got.cpu().numpy(), ref) <= tol, k
    for a, b in zip(g, g_again):
        assert torch.equal(a, b)                       # fixed summation order
    # partial requests
    only_vec = oeq.oeq_radial_bwd(plan, dv, RC, d1, d2, dg, want=("vec",))
    assert only_vec[1] is None and only_vec[2] is None and torch.equal(only_vec[0], g[0])


def test_radial_empty():
    wl = SMALL["tiny_fp64"]
    plan = plan_for(wl)
    vec = torch.zeros(0, 3, dtype=torch.float64, device="cuda")
    W1 = torch.randn(8, 16, dtype=torch.float64, device="cuda")
    W2 = torch.randn(16, plan.n_paths * plan.U, dtype=torch.float64, device="cuda")
    W = oeq.oeq_radial_fwd(plan, vec, RC, W1, W2)
    gW = torch.zeros(0, plan.n_paths, plan.U, dtype=torch.float64, device="cuda")
    gv, g1, g2 = oeq.oeq_radial_bwd(plan, vec, RC, W1, W2, gW)
    torch.cuda.synchronize()
    assert W.shape[0] == 0 and gv.shape == (0, 3)
    assert not g1.cpu().numpy().any() and not g2.cpu().numpy().any()
    # the in-kernel forward and VJP on a graph without edges
    N = 5
    rowptr = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    src = torch.zeros(0, dtype=torch.int32, device="cuda")
    x = torch.randn(N, plan.x_dim, dtype=torch.float64, device="cuda")
    Y = torch.zeros(0, plan.y_dim, dtype=torch.float64, device="cuda")
    g = torch.randn(N, plan.out_dim, dtype=torch.float64, device="cuda")
    W1s, W2s = W1[:, :8].contiguous(), W2[:8].contiguous()
    out = torch.full((N, plan.out_dim), float("nan"), dtype=torch.float64, device="cuda")
    oeq.oeq_tp_conv_fwd_radial(plan, rowptr, src, x, Y, vec, RC, W1s, W2s, out=out)
    res = oeq.oeq_tp_conv_bwd_radial(plan, rowptr, src, x, Y, vec, RC, W1s, W2s, g)
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any()
    assert not res["x"].cpu().numpy().any() and not res["W2"].cpu().numpy().any()


@pytest.mark.slow
def test_radial_full_size_sampled():
    """280,000 edges of the medium workload, hidden width 64, compared on sampled
    edges (the weights and the vector gradient are per edge)."""
    wl = synth.WORKLOADS["mace_medium_fp32"]
    plan = plan_for(wl)
    vec, W1, W2, _ = _problem(wl, plan, 64, 6)
    E, PU = len(vec), plan.n_paths * plan.U
    dv, d1, d2 = (to_dev(a) for a in (vec, W1, W2))
    gW = synth.extra_normal(wl, (E, plan.n_paths, plan.U), 7)
    gWd = to_dev(gW)
    W = oeq.oeq_radial_fwd(plan, dv, RC, d1, d2)
    gv, _, _ = oeq.oeq_radial_bwd(plan, dv, RC, d1, d2, gWd, want=("vec",))
    torch.cuda.synchronize()
    edges = sample(E, 400, 13)
    et = torch.from_numpy(edges).cuda()
    gWs = gW[edges].reshape(len(edges), PU)
    assert rel_l2(W[et].reshape(len(edges), PU).cpu().numpy(), radial.radial_fwd(vec[edges], RC, W1, W2)) <= 1e-5
    rv, _, _ = radial.radial_bwd(vec[edges], RC, W1, W2, gWs)
    assert rel_l2(gv[et].cpu().numpy(), rv) <= 1e-5


@pytest.mark.parametrize("name", ["tiny_fp64", "mace_medium_fp32", "mace_medium_fp64", "mace_large_fp32",
                                  "ragged_u96_f32", "u1_l3_f64", "u8_l1_f32"])
def test_fwd_radial_fused_parity(name):
    """The forward that forms W in the kernel (hidden width 8) against the oracle
    forward on the oracle's radial weights."""
    import oracle
    wl = SMALL[name]
    plan = plan_for(wl)
    d = oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max)
    inp = synth.generate(wl, d.P, d.out_dim, want=("x", "Y", "evec"))
    rng = np.random.default_rng(21)
    dt = wl.np_dtype()
    W1 = rng.standard_normal((8, 8)).astype(dt)
    W2 = rng.standard_normal((8, plan.n_paths * plan.U)).astype(dt)
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "evec")}
    out = torch.full((wl.n_nodes, plan.out_dim), float("nan"), dtype=plan.torch_dtype(), device="cuda")
    oeq.oeq_tp_conv_fwd_radial(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["evec"], RC, to_dev(W1),
                               to_dev(W2), out=out)
    torch.cuda.synchronize()
    Wref = radial.radial_fwd(inp["evec"], RC, W1, W2).reshape(inp["E"], plan.n_paths, plan.U)
    ref = oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], Wref)
    assert rel_l2(out.cpu().numpy(), ref) <= RTOL[wl.dtype]


def _plan_with(wl, env):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        return plan_for(wl)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("name", ["tiny_fp64", "mace_medium_fp32", "mace_medium_fp64", "mace_large_fp32",
                                  "ragged_u96_f32", "u1_l3_f64"])
def test_bwd_radial_fused_parity(name, mode):
    """The VJP with W formed in the kernel (hidden width 8) against the oracle:
    grad_x, grad_Y from the oracle VJP on the oracle's radial weights; grad_vec,
    grad_W1, grad_W2 from the oracle radial backward of the oracle's grad_W."""
    _check_bwd_radial(name, mode, {})


# the other route than the planned one: composed through W where the in-kernel pass
# fits registers, in-kernel where the plan composes (the medium fp64 configuration)
ROUTES = [("mace_medium_fp32", "1"), ("tiny_fp64", "1"), ("u1_l3_f64", "1"), ("mace_medium_fp64", "0")]


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("name,compose", ROUTES)
def test_bwd_radial_routes(name, compose, mode):
    _check_bwd_radial(name, mode, {"OEQ_RAD_COMPOSE": compose})


def _check_bwd_radial(name, mode, env):
    import oracle
    wl = SMALL[name]
    plan = _plan_with(wl, env)
    d = oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max)
    inp = synth.generate(wl, d.P, d.out_dim, want=("x", "Y", "evec", "g"))
    rng = np.random.default_rng(22)
    dt = wl.np_dtype()
    W1 = rng.standard_normal((8, 8)).astype(dt)
    W2 = rng.standard_normal((8, plan.n_paths * plan.U)).astype(dt)
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "evec", "g")}
    print(f"[bwd radial] {name} {mode} {env}", flush=True)
    res = oeq.oeq_tp_conv_bwd_radial(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["evec"], RC,
                                     to_dev(W1), to_dev(W2), dev["g"], mode=mode)
    again = oeq.oeq_tp_conv_bwd_radial(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["evec"], RC,
                                       to_dev(W1), to_dev(W2), dev["g"], mode=mode, want=("vec", "W1", "W2"))
    torch.cuda.synchronize()
    E = inp["E"]
    Wref = radial.radial_fwd(inp["evec"], RC, W1, W2).reshape(E, plan.n_paths, plan.U)
    rx, rY, rW = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], Wref, inp["g"])
    rv, r1, r2 = radial.radial_bwd(inp["evec"], RC, W1, W2, rW.reshape(E, -1))
    tol = RTOL[wl.dtype]
    for k, ref in (("x", rx), ("Y", rY), ("vec", rv), ("W1", r1), ("W2", r2)):
        assert rel_l2(res[k].cpu().numpy(), ref) <= tol, k
    for k in ("vec", "W1", "W2"):
        assert torch.equal(res[k], again[k]), k     # fixed summation order


def test_bwd_radial_rejects_low_Y_degree():
    wl = SMALL["u8_l1_f32"]
    plan = plan_for(wl)
    N, E = 4, 3
    rowptr = torch.tensor([0, 1, 2, 3, 3], dtype=torch.int32, device="cuda")
    src = torch.tensor([1, 2, 0], dtype=torch.int32, device="cuda")
    f = lambda *s: torch.zeros(*s, dtype=torch.float32, device="cuda")
    with pytest.raises(oeq.OeqError, match="UNSUPPORTED"):
        oeq.oeq_tp_conv_bwd_radial(plan, rowptr, src, f(N, plan.x_dim), f(E, plan.y_dim), f(E, 3), RC, f(8, 8),
                                   f(8, plan.n_paths * plan.U), f(N, plan.out_dim))
