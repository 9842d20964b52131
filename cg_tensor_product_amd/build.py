"""Builds liboeq.so (the C-ABI library) in-tree.

Host sources are compiled with g++, the ahead-of-time HIP sources with hipcc for
gfx950, and the kernel template text is embedded as a string for runtime
compilation.  All HIP code is built without packed fp32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liboeq.so")
JITC = os.path.join(PKG, "oeq_jitc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HOST_SOURCES = ["capi.cpp", "capi_graph.cpp", "capi_edge.cpp", "planner.cpp", "cg_tables.cpp", "codegen.cpp", "jit.cpp"]
HIP_SOURCES = ["csr.hip", "noalloc.hip"]
ARCH = "gfx950"
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


# Parts of the kernel template, concatenated in this order after the planner's prelude.
TEMPLATE_PARTS = ["kernels_common.tpl.hip", "kernels_conv.tpl.hip", "kernels_sender.tpl.hip",
                  "kernels_gemm_radial.tpl.hip", "kernels_radial_fused.tpl.hip", "kernels_dbwd.tpl.hip"]


def _embed_template() -> str:
    text = ""
    for part in TEMPLATE_PARTS:
        with open(os.path.join(CSRC, part)) as f:
            text += f.read() + "\n"
    delim = "OEQTPL"
    assert (")" + delim + '"') not in text
    out = os.path.join(BUILD, "kernel_template.cpp")
    body = ("// generated from csrc/kernels_*.tpl.hip\nnamespace oeq {\nextern const char *kKernelTemplate;\n"
            f'const char *kKernelTemplate = R"{delim}(' + text + f'){delim}";\n}}\n')
    old = open(out).read() if os.path.exists(out) else None
    if old != body:
        with open(out, "w") as f:
            f.write(body)
    return out


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    tpl = _embed_template()
    common = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-I" + INCLUDE, "-I" + CSRC,
              "-I" + os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__"]
    jobs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        jobs.append(["g++", *common, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs.append(["g++", *common, "-c", tpl, "-o", os.path.join(BUILD, "kernel_template.o")])
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append([os.path.join(ROCM, "bin", "hipcc"), "-O3", "-fPIC", "-std=c++17",
                     f"--offload-arch={ARCH}", *NO_PACKED_FP32, "-I" + INCLUDE, "-I" + CSRC,
                     "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                sys.stderr.write(r.stdout + r.stderr)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([os.path.join(ROCM, "bin", "hipcc"), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs,
          "-L" + os.path.join(ROCM, "lib"), "-lhiprtc", "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, LIB)
    # the runtime-compiler helper (a separate program: see csrc/jitc_main.cpp); DT_RPATH so
    # that it loads this installation's runtime compiler whatever LD_LIBRARY_PATH holds
    rocm_lib = os.path.join(ROCM, "lib")
    _run(["g++", *common, os.path.join(CSRC, "jitc_main.cpp"), "-o", JITC + ".tmp", "-L" + rocm_lib, "-lhiprtc",
          "-ldl", "-Wl,--disable-new-dtags", "-Wl,-rpath," + rocm_lib])
    os.replace(JITC + ".tmp", JITC)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
