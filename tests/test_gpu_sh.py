"""GPU parity of the Y-from-edge-vectors step against the oracle: the real
spherical harmonics of edge vectors and their gradient, standalone and inside
the forward (evaluated in the kernel) and the VJP (gradient to the vectors)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import RTOL, plan_for, rel_l2, sample, to_dev
from oracle import sphere
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")

NAMES = ["tiny_fp64", "mace_medium_fp32", "mace_medium_fp64", "mace_large_fp32", "u1_l3_f64", "u8_l1_f32",
         "ragged_u96_f32", "ysub_u16_f64"]


def _cols(wl):
    """Columns of the harmonics of degrees 0..max that make up the workload's Y row."""
    return np.concatenate([np.arange(l * l, (l + 1) ** 2) for l in wl.y_degrees])


def _sh(wl, vec):
    return sphere.sh_of_vectors(max(wl.y_degrees), vec)[:, _cols(wl)]


def _sh_grad(wl, vec):
    return sphere.sh_grad_of_vectors(max(wl.y_degrees), vec)[:, _cols(wl), :]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _case(name, special=False):
    wl = SMALL[name]
    d = oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max, y_irreps=wl.y_irreps)
    inp = synth.generate(wl, d.P, d.out_dim, want=("x", "evec", "W", "g"))
    if special:
        # the first edges carry the zero vector, the six axis directions (+-z included), a
        # tiny and a huge vector
        sv = _special_vectors(wl.np_dtype())
        k = min(len(sv), inp["E"])
        inp["evec"][:k] = sv[:k]
    inp["Y"] = _sh(wl, inp["evec"])                                # the oracle's Y of the same vectors
    return wl, d, inp, plan_for(wl)


def _special_vectors(dt):
    # a zero vector, the six axis directions, a tiny and a huge vector
    v = [[0, 0, 0], [1, 0, 0], [-2, 0, 0], [0, 3, 0], [0, -1, 0], [0, 0, 0.5], [0, 0, -4],
         [1e-3, -2e-3, 5e-4], [3e2, 1e2, -2e2]]
    return np.array(v, dtype=dt)


@pytest.mark.parametrize("name", NAMES)
def test_sph_harm_parity(name):
    wl, d, inp, plan = _case(name)
    vec = np.concatenate([inp["evec"], _special_vectors(wl.np_dtype())])
    Y = oeq.oeq_sph_harm(plan, to_dev(vec))
    torch.cuda.synchronize()
    ref = _sh(wl, vec)
    got = Y.cpu().numpy()
    assert rel_l2(got, ref) <= RTOL[wl.dtype]
    # zero vector: exactly Y_00 = 1 (where the plan has degree 0) and 0 elsewhere
    assert np.array_equal(got[len(inp["evec"])], (_cols(wl) == 0).astype(got.dtype))


@pytest.mark.parametrize("name", NAMES)
def test_sph_harm_bwd_parity(name):
    wl, d, inp, plan = _case(name)
    special = _special_vectors(wl.np_dtype())
    vec = np.concatenate([inp["evec"], special])
    gY = synth.extra_normal(wl, (len(vec), plan.y_dim), 3)
    gvec = oeq.oeq_sph_harm_bwd(plan, to_dev(vec), to_dev(gY))
    torch.cuda.synchronize()
    ref = np.einsum("em,emk->ek", gY.astype(np.float64), _sh_grad(wl, vec))
    got = gvec.cpu().numpy()
    assert rel_l2(got, ref) <= RTOL[wl.dtype]
    # the special vectors alone (the six axis directions, +-z included; tiny and huge)
    n = len(inp["evec"])
    assert rel_l2(got[n + 1:], ref[n + 1:]) <= RTOL[wl.dtype]
    assert not got[n].any()                                         # zero vector: zero gradient


@pytest.mark.parametrize("name", NAMES)
def test_fwd_vec_parity(name):
    wl, d, inp, plan = _case(name, special=True)
    print(f"[fwd vec] {name}", flush=True)
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "evec", "W")}
    out = oeq.oeq_tp_conv_fwd_vec(plan, dev["rowptr"], dev["src"], dev["x"], dev["evec"], dev["W"])
    torch.cuda.synchronize()
    ref = oracle.fwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"])
    assert rel_l2(out.cpu().numpy(), ref) <= RTOL[wl.dtype]


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("name", NAMES)
def test_bwd_vec_parity(name, mode):
    wl, d, inp, plan = _case(name, special=True)
    print(f"[bwd vec] {name} {mode}", flush=True)
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "evec", "W", "g")}
    gx, gvec, gW = oeq.oeq_tp_conv_bwd_vec(plan, dev["rowptr"], dev["src"], dev["x"], dev["evec"], dev["W"],
                                           dev["g"], mode=mode)
    torch.cuda.synchronize()
    rx, rY, rW = oracle.bwd(d, inp["rowptr"], inp["src"], inp["x"], inp["Y"], inp["W"], inp["g"])
    rvec = np.einsum("em,emk->ek", rY, _sh_grad(wl, inp["evec"]))
    tol = RTOL[wl.dtype]
    assert rel_l2(gx.cpu().numpy(), rx) <= tol
    assert rel_l2(gW.cpu().numpy(), rW) <= tol
    assert rel_l2(gvec.cpu().numpy(), rvec) <= tol
    k = min(len(_special_vectors(wl.np_dtype())), inp["E"])
    assert rel_l2(gvec[:k].cpu().numpy(), rvec[:k]) <= tol            # the special vectors' edges alone
    # partial request: the vector gradient alone
    _, gv2, _ = oeq.oeq_tp_conv_bwd_vec(plan, dev["rowptr"], dev["src"], dev["x"], dev["evec"], dev["W"], dev["g"],
                                        mode=mode, want=("vec",))
    assert rel_l2(gv2.cpu().numpy(), rvec) <= tol


@pytest.mark.slow
def test_vec_full_size_sampled():
    """mace_medium_fp32 at full size from edge vectors, compared on sampled rows and edges."""
    wl = synth.WORKLOADS["mace_medium_fp32"]
    d = oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max)
    inp = synth.generate(wl, d.P, d.out_dim, want=("x", "evec", "W", "g"))
    plan = plan_for(wl)
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "evec", "W", "g")}
    out = oeq.oeq_tp_conv_fwd_vec(plan, dev["rowptr"], dev["src"], dev["x"], dev["evec"], dev["W"])
    gx, gvec, gW = oeq.oeq_tp_conv_bwd_vec(plan, dev["rowptr"], dev["src"], dev["x"], dev["evec"], dev["W"],
                                           dev["g"])
    torch.cuda.synchronize()
    tol = RTOL[wl.dtype]
    rows = sample(wl.n_nodes, 16, 11)
    e = synth.edges_of_rows(inp["rowptr"], rows)
    rp, sr, e = synth.subgraph(inp["rowptr"], inp["src"], e)
    Ye = sphere.sh_of_vectors(wl.y_lmax, inp["evec"][e])
    ref = oracle.fwd(d, rp, sr, inp["x"], Ye, inp["W"][e], rows=rows)
    assert rel_l2(out[torch.from_numpy(rows).cuda()].cpu().numpy(), ref) <= tol
    edges = sample(inp["E"], 200, 12)
    rp, sr, e = synth.subgraph(inp["rowptr"], inp["src"], edges)
    Ye = sphere.sh_of_vectors(wl.y_lmax, inp["evec"][e])
    rW, rY = oracle.bwd_edges(d, rp, sr, inp["x"], Ye, inp["W"][e], inp["g"])
    rvec = np.einsum("em,emk->ek", rY, sphere.sh_grad_of_vectors(wl.y_lmax, inp["evec"][e]))
    ei = torch.from_numpy(edges).cuda()
    assert rel_l2(gW[ei].cpu().numpy(), rW) <= tol
    assert rel_l2(gvec[ei].cpu().numpy(), rvec) <= tol
