import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity cases (several seconds of oracle work)")


def pytest_sessionstart(session):
    # Load what is built; build only what is missing (hipcc and gcc are on
    # both the build host and the GPU host).
    import oracle
    oracle.build(force=False)
    lib = os.path.join(ROOT, "speculative_decoding_argmax_amd", "lib", "libmtp.so")
    if not os.path.exists(lib):
        from speculative_decoding_argmax_amd import build
        build.build()


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle
