"""Host checks of the seeded graph generator: the receiver-sorted CSR it emits,
distinct senders without self-loops by default, and self-loops plus repeated
(s, r) edges in multigraph mode (the edge cases the kernels must accept)."""
import numpy as np

import synth
from test_gpu_parity import EDGE_CASES, MULTI
from helpers import inputs


def _edges(inp):
    rp, src = inp["rowptr"], inp["src"]
    recv = np.repeat(np.arange(len(rp) - 1), np.diff(rp))
    return recv, src


def test_default_graph_has_distinct_senders_and_no_self_loops():
    wl = synth.WORKLOADS["tiny_fp64"]
    _, inp = inputs(wl, want=())
    recv, src = _edges(inp)
    assert not (recv == src).any()
    assert len(set(zip(recv.tolist(), src.tolist()))) == len(src)
    for r in range(wl.n_nodes):
        row = src[inp["rowptr"][r]:inp["rowptr"][r + 1]]
        assert np.all(np.diff(row) > 0)


def test_multigraph_cases_hold_self_loops_duplicates_and_empty_rows():
    for name in MULTI:
        wl = EDGE_CASES[name]
        _, inp = inputs(wl, want=())
        recv, src = _edges(inp)
        pairs = list(zip(recv.tolist(), src.tolist()))
        assert (recv == src).sum() >= 5, name                       # self-loops
        assert len(pairs) - len(set(pairs)) >= 50, name             # repeated (s, r) edges
        assert (np.diff(inp["rowptr"]) == 0).any(), name            # receivers without edges
        assert np.all(np.diff(inp["rowptr"]) >= 0) and inp["rowptr"][0] == 0
        assert src.min() >= 0 and src.max() < wl.n_nodes
        for r in range(wl.n_nodes):
            row = src[inp["rowptr"][r]:inp["rowptr"][r + 1]]
            assert np.all(np.diff(row) >= 0)                        # sorted inside the row
