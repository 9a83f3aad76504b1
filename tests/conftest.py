import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU statistics")


def _ensure_built():
    """Build a library only when nothing is built yet (build() always rebuilds)."""
    from oracle import build as ob
    from synth import build as sb
    if not os.path.exists(ob.LIB):
        ob.build()
    if not os.path.exists(sb.LIB):
        sb.build()
    try:
        from verify_row_top_amd import build as vb
    except ImportError:
        return
    if not os.path.exists(vb.LIB):
        vb.build()


_ensure_built()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")
