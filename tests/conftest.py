import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(params=["dot", "mfma", "mfma1"])
def decode_kernel(request):
    """Run a test under each form of the INT8/FP8 decode kernel (v_dot2,
    two-pass and one-pass matrix-core), restoring the automatic choice
    afterwards."""
    from paged_int8_kv_amd import binding as B
    B.kv8_set_decode_kernel({"dot": B.DECODE_DOT, "mfma": B.DECODE_MFMA,
                             "mfma1": B.DECODE_MFMA_ONEPASS}[request.param])
    yield request.param
    B.kv8_set_decode_kernel(B.DECODE_AUTO)
