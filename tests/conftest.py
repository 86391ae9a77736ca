import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case, minutes of CPU work")


def pytest_sessionstart(session):
    """Build what is missing (never rebuild what is there): the oracle's shared library and,
    when the HIP toolchain is present, libptg.so and its test builds."""
    import importlib
    oracle = importlib.import_module("oracle")
    oracle.build(force=False)
    from pipelined_tiled_gemm_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    for v in build.VARIANTS:
        if not os.path.exists(build.variant_path(v)):
            build.build(variant=v)
