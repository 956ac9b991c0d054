import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (oracle at large sizes)")


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return True


def pytest_sessionfinish(session, exitstatus):
    """With CPLA_MARGINS_OUT set, write the worst error of every compared output as
    a fraction of its tolerance (1.0 = at the bound), one line per (test, output)."""
    out = os.environ.get("CPLA_MARGINS_OUT")
    if not out:
        return
    mod = sys.modules.get("_parity")
    if mod is None or not mod.MARGINS:
        return
    with open(out, "w") as f:
        for (test, name), r in sorted(mod.MARGINS.items(), key=lambda kv: -kv[1]):
            f.write(f"{r:8.4f}  {test}  {name}\n")
