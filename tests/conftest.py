import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path)")


def _built(path):
    return os.path.exists(os.path.join(ROOT, path))


@pytest.fixture(scope="session", autouse=True)
def _libraries_built():
    """Tests load what is built; they build a part only when it is missing."""
    if not _built("oracle/libzo.so"):
        import oracle
        oracle.build()
    if not (_built("synth/libsynth_host.so") and _built("synth/libsynth_dev.so")):
        import synth.build
        synth.build.build()
    if not _built("sharded_optimizer_step_zero_amd/libzeroshard.so"):
        import __graft_entry__
        __graft_entry__.build_product()
    if not _built("tests/c_abi/abi_check"):
        from c_abi import build as c_abi_build
        c_abi_build.build()
    yield
