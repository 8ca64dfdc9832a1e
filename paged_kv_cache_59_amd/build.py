"""Build the HIP library ``libpagedkv.so`` in-tree for gfx950 with hipcc.

Usage: ``python -m paged_kv_cache_59_amd.build [--trace | --valu]`` (or ``build()``).
Every call recompiles.  Objects go to ``_build/`` at the repository root; the
shared library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
TRACE_LIB_PATH = os.path.join(PKG, "libpagedkv_trace.so")
# measurement builds: the same library with one compile-time switch
VARIANTS = {
    # the decode kernel also writes per-worker timestamps at the start of
    # its workspace (the benchmark's --trace mode)
    "trace": "-DPA_DECODE_TRACE",
    # the decode kernel forms q.K and P.V with v_dot2_f32_f16 on the vector
    # ALUs instead of v_mfma_f32_4x4x4f16 (the benchmark's --decode-variant)
    "valu": "-DPA_DECODE_VALU",
}
ARCH = "gfx950"

SOURCES = ["pa_api.cpp", "pa_cache_ops.hip", "pa_decode.hip", "pa_prefill.hip",
           "pa_prefix.hip", "pa_probe.hip", "pa_block_manager.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep single-lane atomics as written: the atomic optimizer rewrites them
    # into a form whose result is awaited at once, stalling the decode pipeline
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; drop that noise
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def check_no_scratch(remarks: str) -> str:
    """Raise if a kernel's resource-usage remarks report scratch use; else
    a one-line summary."""
    name, kernels, bad = None, 0, []
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
            kernels += 1
        elif "ScratchSize [bytes/lane]:" in line:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0].strip())
            if size:
                bad.append(f"{name}: {size} bytes/lane")
    if bad:
        raise RuntimeError("kernels using scratch memory:\n" + "\n".join(bad))
    return f"{kernels} device functions, none using scratch memory"


def variant_lib_path(variant: str) -> str:
    return os.path.join(PKG, f"libpagedkv_{variant}.so")


def build(verbose: bool = False, trace: bool = False, variant: str | None = None) -> str:
    """Build libpagedkv.so; with ``variant`` (or ``trace``, for "trace") a
    measurement build libpagedkv_<variant>.so instead (VARIANTS)."""
    if trace:
        variant = "trace"
    if variant is not None and variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    out_dir = os.path.join(BUILD_DIR, variant) if variant else BUILD_DIR
    lib_path = variant_lib_path(variant) if variant else LIB_PATH
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        # the resource-usage remarks let the build refuse kernels that spill
        # to scratch memory (a register array indexed at run time, or too
        # many live values): every kernel here is meant to run without it
        remarks = [] if src.endswith(".cpp") else ["-Rpass-analysis=kernel-resource-usage"]
        defs = [VARIANTS[variant]] if variant else []
        cmds.append([HIPCC, *FLAGS, *defs, *lang, *remarks, "-c", os.path.join(CSRC, src), "-o",
                     obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    scratch = check_no_scratch("\n".join(outs))
    outs = [o for o in outs if "kernel-resource-usage" not in o] + [scratch]
    tmp = lib_path + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, lib_path)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv,
          variant="trace" if "--trace" in sys.argv else "valu" if "--valu" in sys.argv else None)
