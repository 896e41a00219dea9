import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # a fresh checkout has no built library: build it once (hipcc cross-compiles
    # gfx950 without a GPU); an existing build is used as it is
    lib = os.path.join(ROOT, "paged_fp8_split_amd", "libpfs.so")
    if not os.path.exists(lib):
        from paged_fp8_split_amd import build

        build.build()
