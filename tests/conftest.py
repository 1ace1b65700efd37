import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_host_libs():
    # Host-side libraries (generator, oracle) are built here if absent; the GPU
    # library is only built by __graft_entry__.build().
    from synth import build as sb
    from oracle import build as ob
    if not os.path.exists(sb.LIB):
        sb.build()
    if not os.path.exists(ob.LIB):
        ob.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")
