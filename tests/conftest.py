import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run through the C ABI")


def pytest_sessionfinish(session, exitstatus):
    path = os.environ.get("GDN_ERR_LOG")
    if not path:
        return
    import json

    import gpu_util

    with open(path, "a") as f:
        for test, what, err, eerr, tol in gpu_util.RECORD:
            f.write(json.dumps({"test": test, "what": what, "normwise": err, "elementwise": eerr, "gate": tol}) + "\n")
