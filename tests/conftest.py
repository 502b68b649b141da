import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # CSA_TEST_LIB runs the tests against another build of the library (the
    # host-sanitised one built by tests/test_abi_asan.py)
    if os.environ.get("CSA_TEST_LIB"):
        from sparse_attention_17_amd import _lib
        _lib.LIB_PATH = os.environ["CSA_TEST_LIB"]


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def lib():
    """The built HIP library (built here if it is missing)."""
    from sparse_attention_17_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_17_amd import build
        build.build()
    return _lib.load()
