import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionfinish(session, exitstatus):
    """Write every code/scale comparison of the session (tests/parity.py
    RECORDS) as JSON lines to the file KVQ_PARITY_REPORT names, if any."""
    path = os.environ.get("KVQ_PARITY_REPORT")
    mod = sys.modules.get("tests.parity")
    if not path or mod is None:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        for r in mod.RECORDS:
            f.write(json.dumps(r) + "\n")
