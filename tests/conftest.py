import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) HIP device")


def pytest_sessionfinish(session, exitstatus):
    """With SSM_PARITY_MARGINS set, write the parity margins the GPU tests observed (see
    tests/gpu_common.py) to that JSON file."""
    path = os.environ.get("SSM_PARITY_MARGINS")
    mod = sys.modules.get("tests.gpu_common")
    if not path or mod is None or not mod.MARGINS:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"exitstatus": int(exitstatus), "tests": mod.MARGINS}, f, indent=1)
        f.write("\n")
