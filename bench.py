#!/usr/bin/env python3
"""Throughput of the fused UVU CG tensor-product convolution on one MI355X.

One step = one forward plus one full VJP (x, Y and W gradients) over the
5,000-node / 280,000-edge receiver-sorted synthetic graph of degree 56 with node
irreps 128x0e+128x1o, Y of degrees 0..3 and all 13 paths with l3 <= 3, in fp32
(the workload of "Receiver-streaming convolutions for channel-wise UVU tensor
products", benchmark paragraph).  Inputs are resident in device memory before
the timed region; graph construction and planning are outside it.

Prints one JSON line: edges/s for the step, the step's algorithmic HBM GB/s, a
roofline entry for the dominant kernel (its average duration from HIP events on
the stream it runs on) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure


def algorithmic_bytes(wl, P, out_dim, E):
    """Bytes the method must move once: inputs read and outputs written.
    Re-reads of x and grad_out rows from cache are not counted."""
    s = 8 if wl.dtype == "f64" else 4
    N = wl.n_nodes
    W = E * P * wl.U * s
    Y = E * wl.y_dim * s
    x = N * wl.x_dim * s
    o = N * out_dim * s
    csr = (N + 1) * 4 + E * 4
    fwd = W + Y + x + o + csr
    vjp = (W + Y + x + o + csr) + (W + Y + x)       # read W,Y,x,g,CSR; write gW,gY,gx
    hvp = (W + Y + x + o + csr) + (W + Y + o)       # read W,Y,v,g,CSR; write dW,dY,dg
    # every tangent: read x,Y,W,g and gg_x,gg_Y,gg_W, CSR; write dx,dY,dW,dg
    dbwd = (2 * (W + Y + x) + o + csr) + (W + Y + x + o)
    return {"fwd": fwd, "vjp": vjp, "hvp": hvp, "dbwd": dbwd}


def measured_traffic(workload, kernel, code_key):
    """HBM bytes per launch of `kernel` from the counter summary under profiles/
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or None if
    there is none for these exact kernels (the code-object hash must match)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic:"):
                rec = json.loads(line[len("traffic:"):])
                if rec.get("code_key") == code_key and kernel in rec.get("bytes_per_launch", {}):
                    return rec["bytes_per_launch"][kernel]
    return None


def stream_reference(torch, nbytes=2 << 30):
    """Same-box context for the HBM figures: a plain device-to-device copy of
    2 GiB (bytes read + written per second), best of 6."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)

    def best_ms(fn):
        best = float("inf")
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    copy_ms = best_ms(lambda: b.copy_(a))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBps": 2 * nbytes / (copy_ms * 1e-3) / 1e9, "bytes": 2 * nbytes}


def side_rows(torch, oeq, plan, dev, N, E, ab, reps=10):
    """Mean duration of the other rows of the hot path on the same inputs (each
    call bracketed by HIP events on the current stream): the deterministic VJP,
    the Hessian-vector product (tangent on x only) and the double backward with
    all three tangents.  Context only: the step is forward + atomic VJP."""
    dt = plan.torch_dtype()
    v = torch.randn(N, plan.x_dim, dtype=dt, device="cuda")
    grads = (torch.empty(N, plan.x_dim, dtype=dt, device="cuda"), torch.empty(E, plan.y_dim, dtype=dt, device="cuda"),
             torch.empty(E, plan.n_paths, plan.U, dtype=dt, device="cuda"))
    outs = {"x": grads[0], "Y": grads[1], "W": grads[2],
            "grad_out": torch.empty(N, plan.out_dim, dtype=dt, device="cuda")}
    hvp_outs = {k: outs[k] for k in ("Y", "W", "grad_out")}

    def ws(mode):
        n = oeq.oeq_workspace_size(plan, N, E, mode)
        if not n:
            return None
        raw = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
        off = (-raw.data_ptr()) % 256
        return raw[off:off + n]

    wsd, wsa = ws("deterministic"), ws("atomic")
    # the tangents of Y and W: copies of Y and W (the cost does not depend on their values, but
    # they must be buffers of their own, or their loads would hit the cache lines of Y and W)
    ggY, ggW = dev["Y"].clone(), dev["W"].clone()
    calls = {
        "vjp_deterministic": (ab["vjp"], lambda: oeq.oeq_tp_conv_bwd(
            plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"], mode="deterministic",
            out=grads, workspace=wsd)),
        "hvp": (ab["hvp"], lambda: oeq.oeq_tp_conv_dbwd(
            plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"], gg_x=v, out=hvp_outs,
            workspace=wsa)),
        "dbwd_all_tangents": (ab["dbwd"], lambda: oeq.oeq_tp_conv_dbwd(
            plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"], gg_x=v, gg_Y=ggY,
            gg_W=ggW, out=outs, workspace=wsa)),
    }
    res = {}
    for name, (nbytes, fn) in calls.items():
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        res[name] = {"ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes, "edges_per_s": E / (ms * 1e-3)}
    del v, grads, outs, wsd, wsa, ggY, ggW
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, d, inp, target_s=10.0, single_s=4.0):
    """The oracle (fp64 loops, OpenMP over independent rows) on the same
    workload: forward of every receiver and the full VJP (W and Y gradients of
    every edge, x gradient of every sender), repeated until about target_s of
    CPU time, on all the threads the oracle uses.  Then the forward alone on one
    thread over the first receivers' rows, about single_s.  Inputs are converted
    to fp64 before the clock starts."""
    import oracle

    x, Y, W, g = (np.ascontiguousarray(inp[k], dtype=np.float64) for k in ("x", "Y", "W", "g"))
    rp, sr = inp["rowptr"], inp["src"]
    reps, t = 0, 0.0
    while t < target_s and reps < 50:
        t0 = time.perf_counter()
        oracle.fwd(d, rp, sr, x, Y, W)
        oracle.bwd_edges(d, rp, sr, x, Y, W, g)
        oracle.bwd_gx(d, rp, sr, Y, W, g)
        t += time.perf_counter() - t0
        reps += 1
    threads = oracle.num_threads()
    # one thread: the forward over the first receivers' rows (a prefix of the CSR)
    oracle.set_num_threads(1)
    rows, t1, e1 = 250, 0.0, 0
    while t1 < single_s and rows <= wl.n_nodes:
        rpp = rp[:rows + 1]
        ne = int(rpp[-1])
        t0 = time.perf_counter()
        oracle.fwd(d, rpp, sr[:ne], x, Y[:ne], W[:ne])
        t1 += time.perf_counter() - t0
        e1 += ne
        rows *= 2
    oracle.set_num_threads(threads)
    return {"value": reps * inp["E"] / t, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole workload ({inp['E']} edges): forward + VJP, {reps} repetition(s), "
                      f"{t:.1f} s in total", "cpu_model": cpu_model(),
            "cpus_in_affinity": len(os.sched_getaffinity(0)),
            "single_thread_fwd": {"value": e1 / t1, "unit": "edges/s", "edges": e1, "seconds": t1,
                                  "sample": "the forward over the first 250, 500, ... receivers' rows, one thread"}}


def fresh_plan_check(torch, oeq, wl, plan, dev, out, reps=20):
    """Forward time of the plan compiled again by oeq_plan_create in this process (a
    process that has loaded torch and its own ROCm libraries), against the plan loaded
    from the code-object cache; once through the compiler helper and once with the
    compiler in this process.  Both timed with HIP events, interleaved."""
    import shutil
    import tempfile

    def fwd_ms(p):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            oeq.oeq_tp_conv_fwd(p, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], out=out)
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    res = {}
    for name, env in (("helper", {}), ("in_process", {"OEQ_JIT_IN_PROCESS": "1"})):
        tmp = tempfile.mkdtemp(prefix="oeq_fresh_")
        old = {k: os.environ.get(k) for k in ("OEQ_CACHE_DIR", "OEQ_JIT_IN_PROCESS")}
        os.environ.update({"OEQ_CACHE_DIR": tmp, **env})
        try:
            t0 = time.perf_counter()
            p2 = oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype)
            compile_s = time.perf_counter() - t0
        finally:
            for k, v in old.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        fwd_ms(p2), fwd_ms(plan)  # load and warm both
        fresh_ms, cached_ms = [], []
        for _ in range(3):
            fresh_ms.append(fwd_ms(p2))
            cached_ms.append(fwd_ms(plan))
        cached_file = os.path.join(ROOT, "cg_tensor_product_amd", "jitcache", plan.code_key + ".hsaco")
        fresh_file = os.path.join(tmp, p2.code_key + ".hsaco")
        same = (os.path.exists(cached_file) and os.path.exists(fresh_file)
                and open(cached_file, "rb").read() == open(fresh_file, "rb").read())
        res[name] = {"compile_s": compile_s, "fwd_ms": float(np.median(fresh_ms)),
                     "cached_fwd_ms": float(np.median(cached_ms)),
                     "ratio": float(np.median(fresh_ms) / np.median(cached_ms)),
                     "same_code_object_bytes": bool(same)}
        del p2
        shutil.rmtree(tmp, ignore_errors=True)
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mace_medium_fp32")
    ap.add_argument("--mode", default="atomic", choices=["atomic", "deterministic"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", default="auto", choices=["auto", "receiver", "sender"],
                    help="schedule of both passes: the plan's data-movement choice per pass (auto), or forced")
    ap.add_argument("--no-side-rows", action="store_true",
                    help="skip timing the deterministic VJP, HVP and all-tangent double backward")
    ap.add_argument("--fresh-plan", action="store_true",
                    help="also compile the plan again in this process (empty code-object cache) and time "
                         "its forward beside the cached plan's: through the compiler helper (the default) "
                         "and with the compiler loaded in this process (OEQ_JIT_IN_PROCESS=1)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device-to-device 3 times (a plain copy kernel of known size, "
                         "to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path runs on a single MI355X "
              "(see the sharding paragraph of the design notes); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import cg_tensor_product_amd as oeq
    import oracle
    import synth

    wl = synth.by_name(args.workload)
    d = oracle.Desc(wl.x_irreps, wl.y_lmax, wl.l3_max, y_irreps=wl.y_irreps, out_irreps=wl.out_irreps)
    inp = synth.generate(wl, d.P, d.out_dim, want=("x", "Y", "W", "g"))
    E, N = inp["E"], wl.n_nodes
    torch.cuda.set_device(0)
    # (a plan missing from the code-object cache is compiled in a child process; see Plan)
    plan = oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype, y_irreps=wl.y_irreps, out_irreps=wl.out_irreps)
    dev = {k: torch.from_numpy(inp[k]).cuda() for k in ("rowptr", "src", "x", "Y", "W", "g")}
    dt = plan.torch_dtype()
    out = torch.empty(N, plan.out_dim, dtype=dt, device="cuda")
    grads = (torch.empty(N, plan.x_dim, dtype=dt, device="cuda"),
             torch.empty(E, plan.y_dim, dtype=dt, device="cuda"),
             torch.empty(E, plan.n_paths, plan.U, dtype=dt, device="cuda"))
    ws = None
    nbytes = oeq.oeq_workspace_size(plan, N, E, args.mode)
    if nbytes:
        raw = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
        off = (-raw.data_ptr()) % 256
        ws = raw[off:off + nbytes]

    # the plan's data-movement model picks each pass's schedule; the sender view of the
    # graph is graph preparation (like the CSR), built before the timed region
    choice = plan.schedule()
    sched_f = choice["fwd"] if args.schedule == "auto" else args.schedule
    sched = choice["bwd"] if args.schedule == "auto" else args.schedule
    view = oeq.oeq_sender_view(dev["rowptr"], dev["src"]) if "sender" in (sched, sched_f) else None
    ws_sender = None
    if sched == "sender":
        nb = oeq.oeq_workspace_size(plan, N, E, "atomic")
        if nb:
            raw_s = torch.empty(nb + 256, dtype=torch.uint8, device="cuda")
            ws_sender = raw_s[(-raw_s.data_ptr()) % 256:][:nb]

    def fwd():
        if sched_f == "sender":
            oeq.oeq_tp_conv_fwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], out=out)
        else:
            oeq.oeq_tp_conv_fwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], out=out)

    def vjp():
        if sched == "sender":
            oeq.oeq_tp_conv_bwd_sender(plan, view, dev["x"], dev["Y"], dev["W"], dev["g"], out=grads,
                                       workspace=ws_sender)
        else:
            oeq.oeq_tp_conv_bwd(plan, dev["rowptr"], dev["src"], dev["x"], dev["Y"], dev["W"], dev["g"],
                                mode=args.mode, out=grads, workspace=ws)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        fwd()
        vjp()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b, c in ev:
        a.record(stream)
        fwd()
        b.record(stream)
        vjp()
        c.record(stream)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    vjp_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))

    fresh = fresh_plan_check(torch, oeq, wl, plan, dev, out) if args.fresh_plan else None

    ab = algorithmic_bytes(wl, d.P, d.out_dim, E)
    ms_step = total / args.steps * 1e3
    step_bytes = ab["fwd"] + ab["vjp"]
    dom, dom_ms, dom_bytes = ("vjp", vjp_ms, ab["vjp"]) if vjp_ms >= fwd_ms else ("fwd", fwd_ms, ab["fwd"])
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    vjp_kernel = "oeq_bwd_sender" if sched == "sender" else (
        "oeq_bwd_atomic" if args.mode == "atomic" else "oeq_bwd_rows")
    kname = {"fwd": "oeq_fwd_sender" if sched_f == "sender" else "oeq_fwd", "vjp": vjp_kernel}[dom]
    traffic = measured_traffic(wl.name, kname, plan.code_key)
    res = {
        "metric": "edges/s and achieved HBM GB/s, fused CG-TP conv fwd+VJP, 5k nodes/280k edges",
        "value": E / (ms_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "nodes": N, "edges": E, "degree": wl.degree,
                   "x_irreps": "+".join(f"{m}x{l}{'e' if p > 0 else 'o'}" for m, l, p in wl.x_irreps),
                   "y_lmax": wl.y_lmax, "paths": d.P,
                   **({"out_irreps": "+".join(f"{m}x{l}{'e' if p > 0 else 'o'}" for m, l, p in wl.out_irreps)}
                      if wl.out_irreps else {}),
                   "step": f"forward ({sched_f}-stationary) + VJP ("
                           + ("sender-stationary" if sched == "sender" else f"receiver-stationary, {args.mode} x-gradient")
                           + ")"},
        "achieved_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "kernels": {
            "fwd": {"ms": fwd_ms, "GBps": ab["fwd"] / (fwd_ms * 1e-3) / 1e9, "bytes": ab["fwd"],
                    "edges_per_s": E / (fwd_ms * 1e-3)},
            "vjp": {"ms": vjp_ms, "GBps": ab["vjp"] / (vjp_ms * 1e-3) / 1e9, "bytes": ab["vjp"],
                    "edges_per_s": E / (vjp_ms * 1e-3)},
        },
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "cpu_baseline": None,
    }
    if not args.no_side_rows:
        res["side_rows"] = side_rows(torch, oeq, plan, dev, N, E, ab)
    if fresh is not None:
        res["fresh_plan"] = fresh
    res["stream_reference"] = stream_reference(torch)
    # the dominant kernel's algorithmic rate as a fraction of this box's plain copy rate
    res["stream_reference"]["frac_of_copy"] = achieved / res["stream_reference"]["copy_GBps"]
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, d, inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
