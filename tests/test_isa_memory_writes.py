"""Every memory write of the library's GPU code goes through the vector memory path.

Scalar-cache writes (scalar stores and atomics, and the scalar data cache's write-back and
discard) are never used: the assembly of every kernel in the library is searched for them.
The global atomics of the watchdog word and of the dynamic tile queue must be vector
(global) atomics.  CPU only: hipcc cross-compiles.  (This file names the scalar write
instructions it searches for, so no GPU run loads it.)
"""
import os
import re
import shutil
import subprocess

import pytest

from pipelined_tiled_gemm_amd import build

hipcc_missing = shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc")

SCALAR_WRITES = re.compile(
    r"^\s*(s_store_|s_buffer_store|s_scratch_store|s_atomic_|s_buffer_atomic|s_dcache_wb|s_dcache_discard)")


@pytest.mark.skipif(hipcc_missing, reason="needs hipcc")
def test_no_scalar_memory_writes(tmp_path):
    text = ""
    for src in build.DEVICE_SOURCES:
        out = tmp_path / (src + ".s")
        subprocess.run([build.hipcc(), *build.compile_flags(source=src), "-S", "--cuda-device-only",
                        os.path.join(build.CSRC, src), "-o", str(out)],
                       check=True, capture_output=True)
        text += out.read_text() + "\n"
    bad = [line.strip() for line in text.split("\n") if SCALAR_WRITES.match(line)]
    assert not bad, bad[:5]
    # the atomics that exist are vector ones
    assert re.search(r"^\s*global_atomic_", text, re.M), "expected the watchdog's global atomic"
