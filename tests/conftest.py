import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


# Alternative builds for the sanitizer runs (tests/test_sanitizers_cpu.py starts the pin and ABI
# suites in subprocesses against sanitizer-instrumented copies of the oracle and the library).
_lib = os.environ.get("QR_TEST_LIB")
if _lib:
    import fp8_block_scaled_qr_amd as _qr
    _qr.LIB_PATH = _lib
_orc = os.environ.get("QR_TEST_ORACLE_LIB")
if _orc:
    from oracle import build as _ob
    _ob.LIB = _orc
    _ob.SRC = _orc          # the instrumented copy is never rebuilt in place
