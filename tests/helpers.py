"""Shared helpers of the test suite: workload setup, tolerances, comparisons."""
from __future__ import annotations

import numpy as np

import oracle
import synth

# Relative L2 bounds per output tensor, by dtype: 1e-5 for fp32, 1e-12 for fp64.
RTOL = {"f32": 1e-5, "f64": 1e-12}


def rel_l2(got, ref) -> float:
    """||got - ref||_2 / ||ref||_2 in fp64 (total error magnitude over the
    reference magnitude); 0/0 counts as 0."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def oracle_desc(wl: synth.Workload) -> oracle.Desc:
    return oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max, y_irreps=wl.y_irreps, out_irreps=wl.out_irreps)


def inputs(wl: synth.Workload, want=("x", "Y", "W", "g")):
    d = oracle_desc(wl)
    return d, synth.generate(wl, d.P, d.out_dim, want=want)


def to_dev(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def plan_for(wl: synth.Workload, env=None):
    """The plan of a workload; `env` sets planner options (OEQ_* variables) while the
    plan is built (the choices are fixed when it is compiled)."""
    import os

    import cg_tensor_product_amd as oeq
    env = env or {}
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        return oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype, y_irreps=wl.y_irreps,
                        out_irreps=wl.out_irreps)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def sample(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct sorted indices of range(n), always including the ends."""
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    s = set(rng.choice(n, size=k - 2, replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(s))


from synth import edges_of_rows, subgraph  # noqa: E402,F401  (graph plumbing lives with the generator)
