import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Sanitizer runs (CPU only): KDNN_TEST_LIB / ORACLE_TEST_LIB name the
# instrumented builds (`python -m kd_tree_nn_amd.build --sanitize`,
# `python -m oracle.build --sanitize`), loaded instead of the normal ones.
if os.environ.get("KDNN_TEST_LIB"):
    from kd_tree_nn_amd import _lib as _kdnn_lib
    _kdnn_lib.LIBPATH = os.environ["KDNN_TEST_LIB"]
if os.environ.get("ORACLE_TEST_LIB"):
    import oracle.ref as _oracle_ref
    _oracle_ref._LIBPATH = os.environ["ORACLE_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP device); run with -m gpu")
    config.addinivalue_line("markers", "slow: long-running CPU test")
