"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every symbol its header declares, builds the same
path lists and CG tables as the oracle (the two are written independently), and
rejects bad arguments with status codes before touching a device.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
from helpers import oracle_desc

oeq = pytest.importorskip("cg_tensor_product_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRIPLES = [(l1, l2, l3) for l1 in range(4) for l2 in range(4) for l3 in range(4)
           if abs(l1 - l2) <= l3 <= l1 + l2]


def _declared():
    text = open(os.path.join(ROOT, "include", "oeq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oeq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = oeq.lib()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(oeq.EXPORTED)


def test_status_strings():
    lib = oeq.lib()
    for code, name in oeq.STATUS.items():
        assert lib.oeq_status_string(code).decode() == name


@pytest.mark.parametrize("l1,l2,l3", TRIPLES)
def test_planner_tables_equal_oracle(l1, l2, l3):
    got = oeq.oeq_cg_table(l1, l2, l3)
    ref = oracle.cg_real(l1, l2, l3)
    assert np.array_equal(got != 0, ref != 0)          # same sparsity, bit for bit
    assert np.abs(got - ref).max() <= 1e-15


def test_cg_table_rejects_bad_degrees():
    with pytest.raises(oeq.OeqError) as e:
        oeq.oeq_cg_table(1, 1, 3)
    assert e.value.status == 1
    with pytest.raises(oeq.OeqError):
        oeq.oeq_cg_table(4, 0, 4)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_plan_paths_and_dims_equal_oracle(name):
    wl = synth.WORKLOADS[name]
    d = oracle_desc(wl)
    p = oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype)
    en = oracle.enumerate_paths(wl.x_irreps, wl.y_lmax, wl.l3_max)
    got = p.paths()
    assert [(i1, l2, l3, p3) for (i1, _, l2, l3, _, p3) in got] == en
    assert [ob for (*_, ob, _) in got] == list(range(len(en)))
    assert (p.x_dim, p.y_dim, p.out_dim, p.n_paths, p.w_per_edge) == (
        d.x_dim, d.y_dim, d.out_dim, d.P, d.P * d.U)


def test_plan_with_output_irreps_sums_paths():
    # 1o x (0e + 2e) -> 1o: two paths into one output block
    p = oeq.Plan("4x1o", 2, 1, "f32", out_irreps="4x1o")
    assert p.n_paths == 2 and p.out_dim == 12
    assert [t[4] for t in p.paths()] == [0, 0]
    q = oeq.Plan("4x1o", 2, 1, "f32", paths=[(0, 0, 0), (0, 2, 0)], out_irreps="4x1o")
    assert q.paths() == p.paths()


@pytest.mark.parametrize("kw,status", [
    (dict(x_irreps="8x0e+4x1o", y_lmax=2), 2),          # mixed multiplicities
    (dict(x_irreps="8x4e", y_lmax=2), 2),               # degree above 3
    (dict(x_irreps="8x0e", y_lmax=4), 2),               # Y degree above 3
    (dict(x_irreps="8x1o", y_lmax=1, dtype="f16"), 2),  # unsupported dtype
    (dict(x_irreps=(), y_lmax=1), 1),                    # no x blocks
    (dict(x_irreps="8x1o", y_lmax=1, paths=[(0, 1, 0)], out_irreps="8x1o"), 1),  # parity violated
    (dict(x_irreps="8x1o", y_lmax=1, paths=[(0, 1, 0)], out_irreps="8x3o"), 1),  # triangle violated
    (dict(x_irreps="8x1o", y_lmax=1, paths=[(0, 0, 0)]), 1),                     # paths without outputs
    (dict(x_irreps="8x0e", y_lmax=2, lmax_out=1, out_irreps="8x3e"), 1),        # no path survives
    (dict(x_irreps="2048x0e", y_lmax=1), 2),                                     # more than 1024 channels
])
def test_plan_create_errors(kw, status):
    with pytest.raises(oeq.OeqError) as e:
        oeq.Plan(**kw)
    assert e.value.status == status


def _raw_call(plan, N, E, rowptr=16, src=16, x=16, mode=0, ws=None, wsb=0, gx=16):
    lib = oeq.lib()
    P = ctypes.c_void_p
    return lib.oeq_tp_conv_bwd(plan, N, E, P(rowptr) if rowptr else None, P(src) if src else None,
                               P(x) if x else None, P(16), P(16), P(16), P(gx) if gx else None, P(16), P(16),
                               mode, P(ws) if ws else None, wsb, None)


def test_compute_argument_errors_before_any_device_work():
    p = oeq.Plan("8x0e+8x1o", 2, 1, "f64")
    lib = oeq.lib()
    P = ctypes.c_void_p
    assert lib.oeq_tp_conv_fwd(None, 4, 4, P(16), P(16), P(16), P(16), P(16), P(16), None) == 1
    assert lib.oeq_tp_conv_fwd(p.handle, -1, 4, P(16), P(16), P(16), P(16), P(16), P(16), None) == 1
    assert lib.oeq_tp_conv_fwd(p.handle, 0, 4, P(16), P(16), P(16), P(16), P(16), P(16), None) == 1
    assert lib.oeq_tp_conv_fwd(p.handle, 4, 4, None, P(16), P(16), P(16), P(16), P(16), None) == 1
    assert lib.oeq_tp_conv_fwd(p.handle, 4, 4, P(16), P(16), None, P(16), P(16), P(16), None) == 1
    assert lib.oeq_tp_conv_fwd(p.handle, 4, 4, P(16), P(16), P(16), P(16), P(16), None, None) == 1
    assert lib.oeq_tp_conv_fwd(p.handle, 2**31, 4, P(16), P(16), P(16), P(16), P(16), P(16), None) == 2
    # N = 0 with no edges is a valid empty call
    assert lib.oeq_tp_conv_fwd(p.handle, 0, 0, P(16), None, None, None, None, None, None) == 0
    assert _raw_call(p.handle, 4, 4, mode=7) == 1
    assert _raw_call(p.handle, 4, 4, x=None) == 1
    assert _raw_call(p.handle, 4, 4, src=None) == 1
    assert _raw_call(p.handle, 4, 4, mode=1, ws=None) == 3          # deterministic needs a workspace
    assert _raw_call(p.handle, 4, 4, mode=1, ws=4096 + 8, wsb=1 << 20) == 3   # misaligned
    assert "aligned" in lib.oeq_last_error().decode()
    # nothing requested: returns without work
    lib2 = lib.oeq_tp_conv_bwd(p.handle, 4, 4, P(16), P(16), P(16), P(16), P(16), P(16), None, None, None,
                               0, None, 0, None)
    assert lib2 == 0


def test_workspace_size_atomic(monkeypatch):
    # the receiver-stationary VJP (forced: this plan's model prefers the sender-stationary one)
    monkeypatch.setenv("OEQ_SCHEDULE", "rr")
    # one size serves the VJP and the double backward: the latter's two path groups (one per
    # x block) need partial Y-gradient rows
    assert oeq.oeq_workspace_size(oeq.Plan("8x0e+8x1o", 2, 1, "f64"), 64, 1024, "atomic") == 2 * 1024 * 9 * 8
    # one group for both -> no scratch in atomic mode
    monkeypatch.setenv("OEQ_DBWD_GROUPS", "1")
    assert oeq.oeq_workspace_size(oeq.Plan("8x0e+8x1o", 2, 1, "f64"), 64, 1024, "atomic") == 0
    monkeypatch.delenv("OEQ_DBWD_GROUPS")
    # two groups -> per-group partial Y-gradient rows
    monkeypatch.setenv("OEQ_BWD_GROUPS", "2")
    p = oeq.Plan("8x0e+8x1o", 2, 1, "f64")
    monkeypatch.delenv("OEQ_BWD_GROUPS")
    monkeypatch.delenv("OEQ_SCHEDULE")
    assert oeq.oeq_workspace_size(p, 64, 1024, "atomic") == 2 * 1024 * 9 * 8
    assert oeq.oeq_workspace_size(p, 64, 1024, "deterministic") > 1024 * 32 * 8
    b = ctypes.c_size_t()
    assert oeq.lib().oeq_workspace_size(p.handle, 64, 1024, 9, ctypes.byref(b)) == 1
    assert oeq.lib().oeq_workspace_size(None, 64, 1024, 0, ctypes.byref(b)) == 1


def test_generated_source_has_no_packed_fp32_and_caches(tmp_path, monkeypatch):
    """The emitted kernels compile for gfx950 on the host (runtime compiler, no
    device), and the code object lands in the cache directory."""
    import subprocess
    import sys
    env = dict(os.environ, OEQ_CACHE_DIR=str(tmp_path))
    code = ("import sys; sys.path.insert(0, %r); import cg_tensor_product_amd as m; "
            "m.Plan('16x0e+16x1o', 1, 1, 'f32')" % ROOT)
    subprocess.run([sys.executable, "-c", code], check=True, env=env)
    objs = list(tmp_path.glob("*.hsaco"))
    assert len(objs) == 1
    dis = subprocess.run(["/opt/rocm/llvm/bin/llvm-objdump", "-d", str(objs[0])],
                         capture_output=True, text=True)
    if dis.returncode == 0:
        assert "v_pk_fma_f32" not in dis.stdout and "v_pk_mul_f32" not in dis.stdout
        assert "oeq_fwd" in dis.stdout and "oeq_bwd_atomic" in dis.stdout


def test_plan_from_cache_only_and_compiled_in_the_helper(tmp_path):
    """oeq_plan_create_cached never compiles: with an empty cache it fails with
    OEQ_ERR_JIT and leaves the plan NULL.  Plan() (oeq_plan_create) then compiles in the
    compiler helper, and the code object it leaves in the cache loads here without
    compiling."""
    import subprocess
    import sys
    code = r"""
import ctypes, os, sys
sys.path.insert(0, %r)
import cg_tensor_product_amd as m
L = m.lib()
d = m._Desc()
xs = (m._Irrep * 2)(m._Irrep(4, 0, 1), m._Irrep(4, 1, -1))
d.x_irreps, d.n_x, d.y_lmax, d.lmax_out, d.dtype = xs, 2, 1, 1, m.OEQ_F32
h = ctypes.c_void_p()
assert L.oeq_plan_create_cached(ctypes.byref(d), ctypes.byref(h)) == 5 and not h.value
assert b"not in the cache" in L.oeq_last_error()
assert os.listdir(os.environ["OEQ_CACHE_DIR"]) == [] if os.path.isdir(os.environ["OEQ_CACHE_DIR"]) else True
p = m.Plan("4x0e+4x1o", 1, 1, "f32")
assert [f for f in os.listdir(os.environ["OEQ_CACHE_DIR"]) if f.endswith(".hsaco")] == [p.code_key + ".hsaco"]
assert L.oeq_plan_create_cached(ctypes.byref(d), ctypes.byref(h)) == 0 and h.value
L.oeq_plan_destroy(h)
print("ok")
""" % ROOT
    env = dict(os.environ, OEQ_CACHE_DIR=str(tmp_path / "cache"))
    env.pop("OEQ_JIT_IN_PROCESS", None)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr


def test_plans_compile_the_same_whatever_the_process_loaded(tmp_path):
    """A framework that bundles another ROCm release's compiler library (this PyTorch wheel
    does) loads it into the process; compiled in that process, the runtime compiler used it
    and produced other (on MI355X, slower) code.  oeq_plan_create compiles in its helper, so
    a plan made after importing torch gets exactly the code object of a plan made in a
    process that loaded nothing else."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n%s\nimport cg_tensor_product_amd as m\n"
            "print(m.Plan('32x0e+32x1o', 3, 3, 'f32').code_key)")
    objs = []
    for k, pre in enumerate(("import torch", "")):
        d = tmp_path / f"c{k}"
        env = dict(os.environ, OEQ_CACHE_DIR=str(d))
        env.pop("OEQ_JIT_IN_PROCESS", None)
        r = subprocess.run([sys.executable, "-c", code % (ROOT, pre)], env=env, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append((d / (r.stdout.strip() + ".hsaco")).read_bytes())
    assert objs[0] == objs[1]


def test_tile_form_rows_match_the_tables(tmp_path):
    """The tile-form forward stores, per edge and path, one Y-contracted entry for every
    (m1, m3) that a non-zero CG coefficient reaches: the emitted row sizes equal that count
    taken from the oracle's tables; rows are whole 16-byte vectors, an odd number of them;
    a tile's rows fit the 80 KB LDS budget.  fp64 plans use the tile form by default."""
    import re
    import subprocess
    import sys
    env = dict(os.environ, OEQ_CACHE_DIR=str(tmp_path), OEQ_DUMP_SOURCE="1")
    code = ("import sys; sys.path.insert(0, %r); import cg_tensor_product_amd as m; "
            "m.Plan('4x0e+4x1o+4x2e', 2, 2, 'f64')" % ROOT)
    subprocess.run([sys.executable, "-c", code], check=True, env=env)
    src = next(tmp_path.glob("*.hip")).read_text()
    assert "constexpr bool FWD_LDS = true;" in src
    rows = [tuple(map(int, t)) for t in re.findall(r"static constexpr int KM = (\d+), SM = (\d+), MOFF = (\d+);", src)]
    assert rows, "no tile-form rows emitted"
    want = 0
    xl = [0, 1, 2]
    for (i1, l2, l3, _) in oracle.enumerate_paths(((4, 0, 1), (4, 1, -1), (4, 2, 1)), 2, 2):
        c = oracle.cg_real(xl[i1], l2, l3)
        want += len({(a, k) for a, _, k in np.argwhere(np.abs(c) > 1e-10)})
    assert sum(km for km, _, _ in rows) == want
    moff = 0
    for km, sm, off in rows:
        assert off == moff and sm >= km and sm % 2 == 0 and (sm // 2) % 2 == 1  # fp64: 2 per vector
        moff += sm
    tile = int(re.search(r"constexpr int FWD_MT = (\d+);", src).group(1))
    assert tile == 64 and int(re.search(r"constexpr int FWD_M_ELEMS = (\d+);", src).group(1)) == moff
    assert tile * moff * 8 <= 81920


def test_schedule_model_prefers_moving_the_narrower_rows(monkeypatch):
    """The data-movement model of oeq_plan_schedule, in gathered elements per edge
    and channel, an atomic add counting 6: the receiver-stationary forward gathers
    an x row (x width), the sender-stationary one adds into an output row (6 x
    output width); the VJPs move 7 x width (x gather + atomic x gradient) and the
    output width (g gather)."""
    med = oeq.Plan("128x0e+128x1o", 3, 3, "f32").schedule()       # x width 4, output width 55
    assert med == {"fwd": "receiver", "bwd": "receiver", "move_fwd": [4.0, 330.0], "move_bwd": [28.0, 55.0]}
    wl = synth.WORKLOADS["invariant_fp32"]                          # x width 16, output width 4
    inv = oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype).schedule()
    assert inv == {"fwd": "receiver", "bwd": "sender", "move_fwd": [16.0, 24.0], "move_bwd": [112.0, 4.0]}
    # 0e x 0e -> 0e only: x width 1, output width 1
    one = oeq.Plan("8x0e", 0, 0, "f64").schedule()
    assert one == {"fwd": "receiver", "bwd": "sender", "move_fwd": [1.0, 6.0], "move_bwd": [7.0, 1.0]}
    monkeypatch.setenv("OEQ_SCHEDULE", "sr")
    forced = oeq.Plan("128x0e+128x1o", 3, 3, "f32").schedule()
    assert forced["fwd"] == "sender" and forced["bwd"] == "receiver"


def test_sender_entry_argument_errors_before_any_device_work():
    p = oeq.Plan("8x0e+8x1o", 2, 1, "f64")
    lib = oeq.lib()
    P = ctypes.c_void_p
    f = lib.oeq_tp_conv_fwd_sender
    assert f(None, 4, 4, P(16), P(16), P(16), P(16), P(16), P(16), P(16), None) == 1
    assert f(p.handle, 4, 4, None, P(16), P(16), P(16), P(16), P(16), P(16), None) == 1     # srowptr
    assert f(p.handle, 4, 4, P(16), None, P(16), P(16), P(16), P(16), P(16), None) == 1     # sperm
    assert f(p.handle, 4, 4, P(16), P(16), None, P(16), P(16), P(16), P(16), None) == 1     # sdst
    assert f(p.handle, 4, 4, P(16), P(16), P(16), None, P(16), P(16), P(16), None) == 1     # x
    assert f(p.handle, 4, 4, P(16), P(16), P(16), P(16), P(16), P(16), None, None) == 1     # out
    b = lib.oeq_tp_conv_bwd_sender
    assert b(p.handle, 4, 4, P(16), P(16), None, P(16), P(16), P(16), P(16), P(16), P(16), P(16), None, 0,
             None) == 1
    assert b(p.handle, 4, 4, P(16), P(16), P(16), P(16), P(16), P(16), None, P(16), P(16), P(16), None, 0,
             None) == 1                                                                   # grad_out
    # nothing requested: returns without work
    assert b(p.handle, 4, 4, P(16), P(16), P(16), P(16), P(16), P(16), P(16), None, None, None, None, 0,
             None) == 0
    v = lib.oeq_sender_view
    assert v(4, 4, None, P(16), P(16), P(16), P(16), P(256), 1 << 20, None) == 1          # rowptr
    assert v(4, 4, P(16), P(16), P(16), P(16), None, P(256), 1 << 20, None) == 1          # sdst
    assert v(4, 4, P(16), P(16), P(16), P(16), P(16), None, 0, None) == 3                  # workspace
    assert v(4, 4, P(16), P(16), P(16), P(16), P(16), P(256 + 8), 1 << 20, None) == 3     # misaligned
    assert v(0, 4, P(16), P(16), P(16), P(16), P(16), P(256), 1 << 20, None) == 1         # edges without nodes


def test_radial_argument_errors_before_any_device_work():
    p = oeq.Plan("8x0e+8x1o", 2, 1, "f64")
    lib = oeq.lib()
    P = ctypes.c_void_p
    b = ctypes.c_size_t()
    assert lib.oeq_radial_workspace_size(p.handle, 100, 16, ctypes.byref(b)) == 0 and b.value > 0
    assert lib.oeq_radial_workspace_size(p.handle, 100, 0, ctypes.byref(b)) == 1
    f = lib.oeq_radial_fwd
    ws, nb = P(4096 * 256), b.value
    assert f(None, 100, P(16), 6.0, 16, P(16), P(16), P(16), ws, nb, None) == 1
    assert f(p.handle, 100, P(16), 0.0, 16, P(16), P(16), P(16), ws, nb, None) == 1        # r_cut
    assert f(p.handle, 100, P(16), 6.0, 2000, P(16), P(16), P(16), ws, nb, None) == 2      # hidden width
    assert f(p.handle, 100, None, 6.0, 16, P(16), P(16), P(16), ws, nb, None) == 1         # vec
    assert f(p.handle, 100, P(16), 6.0, 16, P(16), P(16), P(16), None, 0, None) == 3       # workspace
    assert f(p.handle, 100, P(16), 6.0, 16, P(16), P(16), P(16), P(4096 * 256 + 8), nb, None) == 3
    g = lib.oeq_radial_bwd
    assert g(p.handle, 100, P(16), 6.0, 16, P(16), P(16), None, P(16), None, None, ws, nb, None) == 1  # grad_W
    # nothing requested: returns without work
    assert g(p.handle, 100, P(16), 6.0, 16, P(16), P(16), P(16), None, None, None, ws, nb, None) == 0


# ---------------------------------------------------------------------------
# Y described by its irreps
# ---------------------------------------------------------------------------

Y_CASES = [
    ("32x0e+32x1o", "1x0e+1x2e", 3),               # a missing degree (no 1, no 3)
    ("16x0e+16x1o+16x2e", "1x2e+1x0e+1x1e", 3),    # unsorted, with a pseudovector block
    ("8x1o", "1x3o+1x1o", 2),                      # the odd degrees only
]


@pytest.mark.parametrize("xi,yi,l3", Y_CASES)
def test_plan_with_y_irreps_equals_oracle(xi, yi, l3):
    p = oeq.Plan(xi, 0, l3, "f32", y_irreps=yi)
    xt, yt = oeq._irreps(xi), oeq._irreps(yi)
    d = oracle.Desc(xt, 0, l3, y_irreps=yt)
    en = oracle.enumerate_paths(xt, 0, l3, y_irreps=yt)
    got = p.paths()
    # (x block, l1, l2, l3, output block, output parity) against (x block, Y block, l3, parity)
    assert [(i1, l3_, p3) for (i1, _, _, l3_, _, p3) in got] == [(i1, l3_, p3) for (i1, _, l3_, p3) in en]
    assert [l2 for (_, _, l2, *_) in got] == [yt[j][1] for (_, j, _, _) in en]
    assert (p.x_dim, p.y_dim, p.out_dim, p.n_paths) == (d.x_dim, d.y_dim, d.out_dim, d.P)


def test_default_y_equals_the_natural_harmonics():
    a = oeq.Plan("8x0e+8x1o", 3, 3, "f32")
    b = oeq.Plan("8x0e+8x1o", 0, 3, "f32", y_irreps="1x0e+1x1o+1x2e+1x3o")
    assert a.paths() == b.paths() and a.code_key == b.code_key


def test_y_irreps_rejected():
    def status(**kw):
        with pytest.raises(oeq.OeqError) as e:
            oeq.Plan("8x1o", 0, 3, "f32", **kw)
        return e.value.status
    assert status(y_irreps="2x1o") == 2                          # multiplicity above 1
    assert status(y_irreps="1x4e") == 2                          # degree above 3
    assert status(y_irreps="1x3o+1x3o+1x1o") == 2                # 17 values per row
    # an explicit path must respect the product of the parities: 1o x 1e -> 1o, not 1e
    assert status(y_irreps="1x1e", paths=[(0, 0, 0)], out_irreps="8x1e") == 1
    p = oeq.Plan("8x1o", 0, 3, "f32", y_irreps="1x1e", paths=[(0, 0, 0)], out_irreps="8x1o")
    assert p.paths() == [(0, 1, 1, 1, 0, -1)]
    assert status(y_irreps="1x0e", paths=[(0, 1, 0)], out_irreps="8x1o") == 1   # no Y block 1


def test_vector_entry_points_reject_pseudotensor_y():
    # harmonics of a vector cannot fill a 1e block: refused on the host, before any launch
    p = oeq.Plan("8x1o", 0, 2, "f32", y_irreps="1x0e+1x1e")
    fake = ctypes.c_void_p(0x1000)
    st = oeq.lib().oeq_sph_harm(p.handle, 4, fake, fake, None)
    assert st == 2 and b"parity" in oeq.lib().oeq_last_error()
    assert oeq.lib().oeq_sph_harm_bwd(p.handle, 4, fake, fake, fake, None) == 2
    rp = ctypes.c_void_p(0x2000)
    assert oeq.lib().oeq_tp_conv_fwd_vec(p.handle, 2, 4, rp, fake, fake, fake, fake, fake, None) == 2


def test_noalloc_bwd_rejects_scratch_beyond_its_limit():
    # the deterministic VJP of the 5,000-node / 280,000-edge workload needs ~0.58 GB of
    # per-edge rows: refused on the host with the size, before any device call
    wl = synth.WORKLOADS["mace_medium_fp32"]
    p = oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype)
    fake = ctypes.c_void_p(0x1000)
    st = oeq.lib().oeq_tp_conv_bwd_noalloc(p.handle, 5000, 280000, fake, fake, fake, fake, fake, fake, fake, fake,
                                            fake, 1, None)
    assert st == 3
    msg = oeq.lib().oeq_last_error().decode()
    need = int(re.search(r"needs (\d+) bytes", msg).group(1))
    assert "67108864" in msg and need >= 280000 * 512 * 4


def test_workspace_covers_the_sender_view_when_the_vjp_routes_there():
    # the invariant plan's model prefers the sender-stationary VJP: oeq_tp_conv_bwd builds
    # the sender view (srowptr, sperm, sdst and the counting-sort scratch) in its workspace
    wl = synth.WORKLOADS["invariant_fp32"]
    p = oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype)
    assert p.schedule()["bwd"] == "sender"
    N, E = 5000, 280000
    for mode in ("atomic", "deterministic"):
        assert oeq.oeq_workspace_size(p, N, E, mode) >= 4 * (N + 1 + 2 * E)
    assert oeq.oeq_workspace_size(p, N, 0, "atomic") == 0


# UVW products that reduce to the channel-wise one: one-channel x blocks (broadcast)
# and one-channel output blocks (channel sums)
from test_gpu_uvw import CASES as UVW_CASES  # noqa: E402


@pytest.mark.parametrize("name", list(UVW_CASES))
def test_reducible_plans_equal_oracle(name):
    wl = UVW_CASES[name]
    d = oracle_desc(wl)
    p = oeq.Plan(wl.x_irreps, wl.y_lmax, wl.l3_max, wl.dtype, out_irreps=wl.out_irreps)
    assert [(i1, l2, l3, ob) for (i1, _, l2, l3, ob, _) in p.paths()] == [
        (i1, d.path_l2(k), l3, ob) for k, (i1, _j, l3, ob) in enumerate(d.paths)]
    assert (p.x_dim, p.y_dim, p.out_dim, p.n_paths, p.U) == (d.x_dim, d.y_dim, d.out_dim, d.P, d.U)


def test_reducible_plans_take_the_receiver_passes_only(monkeypatch):
    monkeypatch.setenv("OEQ_SCHEDULE", "ss")
    for xi, oi in (("1x0e+16x1o", None), ("16x0e+16x1o", "1x0e+16x1o+1x1e")):
        p = oeq.Plan(xi, 2, 2, "f32", out_irreps=oi)
        assert (p.schedule()["fwd"], p.schedule()["bwd"]) == ("receiver", "receiver")
        lib, P = oeq.lib(), ctypes.c_void_p
        assert lib.oeq_tp_conv_fwd_sender(p.handle, 0, 0, P(16), None, None, None, None, None, None, None) == 2
        assert b"U channels" in lib.oeq_last_error()
        assert lib.oeq_tp_conv_bwd_sender(p.handle, 0, 0, P(16), None, None, None, None, None, None, None, None,
                                          None, None, 0, None) == 2
        assert lib.oeq_tp_conv_fwd_radial(p.handle, 0, 0, P(16), None, None, None, None, 5.0, None, None, None,
                                          None, 0, None) == 2
        assert lib.oeq_tp_conv_bwd_radial(p.handle, 0, 0, P(16), None, None, None, None, 5.0, None, None, None,
                                          None, None, None, None, None, 0, None, 0, None) == 2


def test_reducible_workspace_holds_the_wide_x_gradient_rows(monkeypatch):
    # atomic VJP of a plan with a broadcast x block: x-gradient rows of U channels in every
    # block (64 x (1 + 3) values per node) in the workspace, summed into the caller's rows
    # (one double-backward group: no partial Y-gradient rows besides)
    monkeypatch.setenv("OEQ_DBWD_GROUPS", "1")
    p = oeq.Plan("1x0e+64x1o", 2, 2, "f32")
    assert p.x_dim == 1 + 64 * 3
    assert oeq.oeq_workspace_size(p, 64, 1024, "atomic") == 64 * 256 * 4
    # per-edge rows of the deterministic VJP have the same width
    assert oeq.oeq_workspace_size(p, 64, 1024, "deterministic") >= 1024 * 256 * 4
    # channel sums alone need no x-gradient rows of their own
    q = oeq.Plan("64x0e+64x1o", 2, 2, "f32", out_irreps="1x0e+64x1o+1x1e")
    assert oeq.oeq_workspace_size(q, 64, 1024, "atomic") == 0


@pytest.mark.parametrize("kw", [
    dict(x_irreps="8x0e+4x1o", y_lmax=2),                      # neither U nor one channel
    dict(x_irreps="8x0e+8x1o", y_lmax=2, out_irreps="4x1o"),  # output of 4 channels against U = 8
])
def test_reducible_plan_errors(kw):
    with pytest.raises(oeq.OeqError) as e:
        oeq.Plan(**kw)
    assert e.value.status == 2
