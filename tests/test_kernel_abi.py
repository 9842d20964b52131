"""Host check that every kernel launch passes as many arguments as the kernel
declares.  hipModuleLaunchKernel takes an untyped argument array, so a kernel
whose signature grew without its launch site would read past the array on the
device.  The expected counts come from the compiled code object's own metadata
(llvm-readelf of a plan compiled here, no GPU); the passed counts come from the
argument arrays in the C-ABI sources."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "cg_tensor_product_amd", "csrc")
READELF = "/opt/rocm/llvm/bin/llvm-readelf"


def _kernel_arg_counts(hsaco: str) -> dict:
    notes = subprocess.run([READELF, "--notes", hsaco], capture_output=True, text=True, check=True).stdout
    out = {}
    for block in re.split(r"\n\s+- \.agpr_count", notes)[1:]:
        m = re.search(r"\.name:\s+(\S+)", block)
        if not m or ".args:" not in block:
            continue
        args = block.split(".args:")[1].split(".group_segment_fixed_size")[0]
        kinds = re.findall(r"\.value_kind:\s+(\S+)", args)
        out[m.group(1)] = len([k for k in kinds if not k.startswith("hidden_")])
    return out


def _launch_sites():
    """(kernel name, number of arguments passed) for every launch with a literal name."""
    sites = []
    for fn in sorted(os.listdir(CSRC)):
        if not fn.startswith("capi") or not fn.endswith((".cpp", ".hpp")):
            continue
        src = open(os.path.join(CSRC, fn)).read()
        arrays = {}
        for m in re.finditer(r"void \*(\w+)\[\] = \{([^}]*)\};|launch\(p, \"(\w+)\", [^;]*?, (\w*args)(?:, \w+)?\)", src, re.S):
            if m.group(1):
                arrays[m.group(1)] = len([a for a in m.group(2).split(",") if a.strip()])
            else:
                name, arr = m.group(3), m.group(4)
                if arr in arrays:
                    sites.append((fn, name, arrays[arr]))
    return sites


@pytest.fixture(scope="module")
def counts(tmp_path_factory):
    if not os.path.exists(READELF):
        pytest.skip("llvm-readelf not found")
    d = tmp_path_factory.mktemp("cache")
    env = dict(os.environ, OEQ_CACHE_DIR=str(d))
    code = ("import sys; sys.path.insert(0, %r); import cg_tensor_product_amd as m; "
            "m.Plan('16x0e+16x1o+16x2e', 3, 3, 'f32')" % ROOT)
    subprocess.run([sys.executable, "-c", code], check=True, env=env)
    objs = list(d.glob("*.hsaco"))
    assert len(objs) == 1
    return _kernel_arg_counts(str(objs[0]))


def test_every_literal_launch_matches_its_kernel(counts):
    sites = _launch_sites()
    assert len(sites) >= 15
    for fn, name, n in sites:
        assert name in counts, (fn, name)
        assert counts[name] == n, (fn, name, n, counts[name])


def test_double_backward_passes_match_their_kernels(counts):
    # oeq_tp_conv_dbwd launches every oeq_dbwd_* kernel through one argument array
    src = open(os.path.join(CSRC, "capi.cpp")).read()
    m = re.search(r"auto pass = .*?void \*args\[\] = \{([^}]*)\};", src, re.S)
    n = len([a for a in m.group(1).split(",") if a.strip()])
    names = [k for k in counts if k.startswith("oeq_dbwd_")]
    assert len(names) >= 20
    for k in names:
        assert counts[k] == n, (k, counts[k], n)
