"""pytest configuration: the ``gpu`` marker and shared fixtures."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The HIP library is built in-tree; build it here only if nothing is built yet.
if not os.path.exists(os.path.join(ROOT, "w4a4_gemm_amd", "libnvfp4.so")):
    import importlib.util
    _spec = importlib.util.spec_from_file_location(
        "w4a4_gemm_amd_build", os.path.join(ROOT, "w4a4_gemm_amd", "build.py"))
    _build = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(_build)
    _build.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes)")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
