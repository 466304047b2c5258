import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _build_missing():
    """Build in-tree native libraries that are not built yet (a built
    library is used as it is)."""
    from routed_expert_ffn_amd import LIB_PATH
    from routed_expert_ffn_amd import build as moe_build
    from synth import build as synth_build

    if not os.path.exists(LIB_PATH):
        moe_build.build()
    if not os.path.exists(synth_build.LIB_GPU):
        synth_build.build_gpu()


_build_missing()
