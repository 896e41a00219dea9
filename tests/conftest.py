import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # build (hipcc cross-compiles gfx950 without a GPU) when a library is
    # missing or its sources, headers included, changed since it was built
    from paged_fp8_split_amd import build

    if build.stale():
        build.build()
