import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _use_sanitized_libraries():
    """CPU sanitizer job: BDATTN_SANITIZED_DIR names a folder holding
    libbdattn.so and libbdoracle.so built with sanitizers
    (build.build_sanitized); the bindings load those instead."""
    d = os.environ.get("BDATTN_SANITIZED_DIR")
    if not d:
        return
    from block_diffusion_lm_bdlm_amd import bdattn
    from oracle import build as orc_build
    bdattn.LIB_PATH = os.path.join(d, "libbdattn.so")
    orc_build.LIB = os.path.join(d, "libbdoracle.so")


def pytest_configure(config):
    _use_sanitized_libraries()
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def orc():
    from oracle import build, oracle
    build.build(force=False)
    return oracle
