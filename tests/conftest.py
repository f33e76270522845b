import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    """A fresh checkout has no built library (it is not kept in the history): build it once,
    before any test loads it. hipcc cross-compiles for gfx950 without a GPU; where the library
    is already built (as on a GPU machine that received the built tree) nothing is compiled."""
    from quantized_delta_rule_gdn_amd import build, lib
    if not os.path.exists(lib.LIB_PATH):
        build.build()
