import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# tests/sanitize_host.py runs the CPU tests on sanitizer builds of the library and the oracle
if os.environ.get("PDECODE_SANITIZED_LIB"):
    import paged_kv_decode_08_amd as _pk
    _pk.LIB_PATH = os.environ["PDECODE_SANITIZED_LIB"]
if os.environ.get("PDECODE_SANITIZED_ORACLE"):
    import oracle as _oracle
    _oracle.LIB = os.environ["PDECODE_SANITIZED_ORACLE"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
