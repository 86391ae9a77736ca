"""Builds libptg.so (gfx950) in-tree with hipcc.

    python -m pipelined_tiled_gemm_amd.build      # or build() from Python

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection
disabled (the kernels are written for plain fp32 VALU and MFMA).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libptg.so")
ARCH = "gfx950"
# Each source with its own extra flags.  The GEMM kernels take the backend's latency-oriented
# instruction scheduler (max-ilp): measured 3-4% faster on the batched and grouped workloads,
# under 1% on the others, with the same bits.  The attention kernel keeps the default
# scheduler, which measured 3% faster for it.
SOURCES = {
    "ptg_kernels.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "ptg_attention.hip": [],
    # the one-role dense kernel: its MFMAs are inline asm that fixes the issue order, so it
    # takes the default scheduler
    "ptg_onerole.hip": [],
    "ptg_api.cpp": [],
}
DEVICE_SOURCES = [s for s in SOURCES if s.endswith(".hip")]
# Test builds of the same sources, each a library of its own next to libptg.so (never loaded
# by the package): "delay" pauses pseudo-randomly at every ring handoff (PTG_DELAY_INJECT),
# for the ring stress tests.
VARIANTS = {"delay": ["-DPTG_DELAY_INJECT=1"]}


def variant_path(name: str) -> str:
    return os.path.join(HERE, f"libptg_{name}.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libptg.so")


def compile_flags(extra=(), source=None):
    """hipcc flags; with `source`, that source's own flags are appended."""
    own = SOURCES.get(source, []) if source else []
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), *own, *extra]


def build(verbose: bool = False, extra=(), variant: str = None) -> str:
    """Builds libptg.so, or with `variant` the test build libptg_<variant>.so."""
    cc = hipcc()
    objs = []
    tmpdir = os.path.join(HERE, "_build", variant or "")
    out = variant_path(variant) if variant else LIB
    if variant:
        extra = (*VARIANTS[variant], *extra)
    os.makedirs(tmpdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmpdir, src + ".o")
        cmd = [cc, *compile_flags(extra, src), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        objs.append(obj)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list:
    """The library and every test build."""
    return [build(verbose)] + [build(verbose, variant=v) for v in VARIANTS]


if __name__ == "__main__":
    for path in build_all(verbose="-v" in sys.argv):
        print(path)
