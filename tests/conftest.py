import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


# tests/sanitize_host.py runs this tier with ASan/UBSan-instrumented copies of the oracle
# and of the library's host code; point both loaders at them before anything loads.
if os.environ.get("BSQ_TEST_SANITIZED") == "1":
    import block_scaled_precision_mxfp8_amd as _bsq
    import oracle as _oracle

    _bsq.LIB_PATH = os.path.join(ROOT, "block_scaled_precision_mxfp8_amd", "libbsq_san.so")
    _oracle._LIB = os.path.join(ROOT, "oracle", "liboracle_san.so")
    assert os.path.exists(_bsq.LIB_PATH) and os.path.exists(_oracle._LIB), "build the sanitized copies first"
