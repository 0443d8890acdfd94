import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size GPU parity case")


def pytest_sessionstart(session):
    # On a GPU, every binding call that takes a workspace reads its device-side flags
    # afterwards and raises if a bounded in-kernel wait ran out or a plan check failed.
    try:
        import torch
        if torch.cuda.is_available():
            import linear_attention_rla_amd as rla
            rla.set_check_flags(True)
    except ImportError:
        pass
