"""Rotation equivariance of the GPU path, a property that holds at any size and so
pins the full-size runs beyond the sampled oracle rows.  Rotating every edge vector
by R and every x row block of degree l by the Wigner matrix D_l(R) must rotate each
output block of degree l3 by D_l3(R) (the CG coefficients intertwine the rotations;
"An Efficient Sparse Kernel Generator for O(3)-Equivariant Deep Networks",
abstract).  For the VJP, with grad_out rotated the same way, grad_x rotates like x,
grad_vec like the vectors, and grad_W does not change.  Both sides run on the GPU
(Y from the vectors in the kernel), so the tolerance is the dtype's rounding."""
import numpy as np
import pytest

import oracle
import synth
from helpers import RTOL, plan_for, rel_l2, to_dev
from oracle import sphere
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
oeq = pytest.importorskip("cg_tensor_product_amd")

ANGLES = (0.83, 2.11, -1.37)   # z-y-z Euler angles of a generic rotation


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _rotate_rows(a, U, ls, ang):
    """Rotate a [rows, U * sum(2l+1)] tensor in the channel-major block layout: each
    block of degree l holds [U, 2l+1] per row and maps v -> D_l v."""
    out = np.empty_like(a)
    off = 0
    for l in ls:
        n = 2 * l + 1
        D = sphere.wigner_d_real(l, *ang)
        blk = a[:, off:off + U * n].reshape(a.shape[0], U, n)
        out[:, off:off + U * n] = (blk @ D.T).reshape(a.shape[0], U * n)
        off += U * n
    return out


def _check(wl, tol):
    d = oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max)
    inp = synth.generate(wl, d.P, d.out_dim, want=("x", "evec", "W", "g"))
    plan = plan_for(wl)
    dt = wl.np_dtype()
    R = sphere.rotation(*ANGLES)
    x, vec, W, g = inp["x"], inp["evec"], inp["W"], inp["g"]
    xr = _rotate_rows(x.astype(np.float64), d.U, d.xl, ANGLES).astype(dt)
    vr = (vec.astype(np.float64) @ R.T).astype(dt)
    gr = _rotate_rows(g.astype(np.float64), d.U, d.out_l, ANGLES).astype(dt)
    rp, sr = to_dev(inp["rowptr"]), to_dev(inp["src"])
    Wd = to_dev(W)
    print(f"[equivariance] {wl.name} N={wl.n_nodes} E={inp['E']}", flush=True)
    out = oeq.oeq_tp_conv_fwd_vec(plan, rp, sr, to_dev(x), to_dev(vec), Wd)
    out_r = oeq.oeq_tp_conv_fwd_vec(plan, rp, sr, to_dev(xr), to_dev(vr), Wd)
    gx, gv, gW = oeq.oeq_tp_conv_bwd_vec(plan, rp, sr, to_dev(x), to_dev(vec), Wd, to_dev(g))
    gx_r, gv_r, gW_r = oeq.oeq_tp_conv_bwd_vec(plan, rp, sr, to_dev(xr), to_dev(vr), Wd, to_dev(gr))
    torch.cuda.synchronize()
    out, out_r = out.cpu().numpy().astype(np.float64), out_r.cpu().numpy()
    assert rel_l2(out_r, _rotate_rows(out, d.U, d.out_l, ANGLES)) <= tol
    gx, gv = gx.cpu().numpy().astype(np.float64), gv.cpu().numpy().astype(np.float64)
    assert rel_l2(gx_r.cpu().numpy(), _rotate_rows(gx, d.U, d.xl, ANGLES)) <= tol
    assert rel_l2(gv_r.cpu().numpy(), gv @ R.T) <= tol
    # grad_W is E x P x U (1.9 GB at full size): compared on the device, in float64
    diff = torch.linalg.vector_norm((gW_r - gW).double()) / torch.linalg.vector_norm(gW.double())
    assert float(diff) <= tol
    # the property is not vacuous: the output does change under the rotation
    assert rel_l2(out_r, out) > 1e-2


@pytest.mark.parametrize("name", ["tiny_fp64", "mace_medium_fp64", "mace_large_fp32", "u1_l3_f64", "u8_l1_f32",
                                  "ragged_u96_f32"])
def test_rotation_equivariance(name):
    wl = SMALL[name]
    # rounding of two independent GPU evaluations, each within the parity bar
    _check(wl, 4 * RTOL[wl.dtype])


def test_rotation_equivariance_full_size():
    """The headline workload at full size (5,000 nodes, 280,000 edges, fp32)."""
    _check(synth.WORKLOADS["mace_medium_fp32"], 4 * RTOL["f32"])
