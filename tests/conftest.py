import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # build the host-side helpers only when nothing is built yet
    from synth import build as sb
    from oracle import build as ob
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        sb.build()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        ob.build()
