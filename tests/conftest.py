import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases")


def pytest_sessionstart(session):
    # The tests load the in-tree library; build it once if it is not there.
    lib = os.path.join(ROOT, "online_structured_ffn_amd", "libpop.so")
    if not os.path.exists(lib):
        from online_structured_ffn_amd.build import build
        build()
