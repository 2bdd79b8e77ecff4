import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(params=["dot", "mfma", "mfma1", "sk"])
def decode_kernel(request):
    """Run a test under each form of the INT8/FP8/INT4 decode kernel (v_dot2,
    two-pass, one-pass and stream-K matrix-core): the test helpers pass the
    form as the kernel_form argument of every decode call they make."""
    from paged_int8_kv_amd import binding as B
    from tests import kv8_testutil as U
    U.FORM = {"dot": B.DECODE_DOT, "mfma": B.DECODE_MFMA, "mfma1": B.DECODE_MFMA_ONEPASS,
              "sk": B.DECODE_STREAMK}[request.param]
    yield request.param
    U.FORM = B.DECODE_AUTO
