import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """Writes the near-tie counts the GPU parity tests logged (one record per
    forward checked on computed keys) to $ROUTER_NEAR_TIE_REPORT, if set."""
    path = os.environ.get("ROUTER_NEAR_TIE_REPORT")
    mod = sys.modules.get("gpu_support")
    if not path or mod is None:
        return
    import json
    with open(path, "w") as f:
        json.dump(mod.NEAR_TIE_LOG, f, indent=0)
