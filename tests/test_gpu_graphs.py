"""The entry points are stream-ordered and allocate nothing, so a caller can
capture them into a HIP graph.  The captured forward, VJP (both modes) and double
backward are replayed several times, with eager work and synchronisations
between the replays, and every replay is checked against the eager result."""
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


def _ws(plan, N, E, mode):
    n = oeq.oeq_workspace_size(plan, N, E, mode)
    if n == 0:
        return None
    raw = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    return raw[off:off + n]


@pytest.mark.parametrize("name", ["mace_medium_fp32", "tiny_fp64"])
def test_graph_replays_match_eager(name):
    wl = synth.WORKLOADS[name]
    if wl.n_nodes > 200:
        wl = wl.scaled(n_nodes=150)
    d, inp = inputs(wl, want=("x", "Y", "W", "g", "v"))
    dev = {k: to_dev(inp[k]) for k in ("rowptr", "src", "x", "Y", "W", "g", "v")}
    plan = plan_for(wl)
    N, E = wl.n_nodes, inp["E"]
    dt = plan.torch_dtype()

    def alloc():
        return {
            "out": torch.empty(N, plan.out_dim, dtype=dt, device="cuda"),
            "ga": tuple(torch.empty(s, dtype=dt, device="cuda") for s in
                        ((N, plan.x_dim), (E, plan.y_dim), (E, plan.n_paths, plan.U))),
            "gd": tuple(torch.empty(s, dtype=dt, device="cuda") for s in
                        ((N, plan.x_dim), (E, plan.y_dim), (E, plan.n_paths, plan.U))),
        }

    wsa, wsd = _ws(plan, N, E, "atomic"), _ws(plan, N, E, "deterministic")

    def run(o):
        oeq.oeq_tp_conv_fwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], out=o["out"])
        oeq.oeq_tp_conv_bwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                            out=o["ga"], workspace=wsa)
        oeq.oeq_tp_conv_bwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                            mode="deterministic", out=o["gd"], workspace=wsd)

    eager = alloc()
    run(eager)                       # also loads the code object on this device
    torch.cuda.synchronize()
    ref = {"out": eager["out"].clone(), "ga": [t.clone() for t in eager["ga"]],
           "gd": [t.clone() for t in eager["gd"]]}

    static = alloc()
    for t in (static["out"], *static["ga"], *static["gd"]):
        t.fill_(float("nan"))
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(static)                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(static)
    tol = RTOL[wl.dtype]
    for rep in range(3):
        for t in (static["out"], *static["ga"], *static["gd"]):
            t.fill_(float("nan"))    # every output must be rewritten by the replay
        graph.replay()
        run(eager)                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(static["out"], ref["out"]), rep
        for a, b in zip(static["gd"], ref["gd"]):
            assert torch.equal(a, b), rep            # deterministic mode: bitwise
        assert torch.equal(static["ga"][1], ref["ga"][1]) and torch.equal(static["ga"][2], ref["ga"][2])
        assert rel_l2(static["ga"][0].cpu().numpy(), ref["ga"][0].cpu().numpy()) <= tol
    del graph
    torch.cuda.synchronize()
