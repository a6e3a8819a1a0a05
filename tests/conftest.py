import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path)")


def pytest_sessionfinish(session, exitstatus):
    path = os.environ.get("TREE_ATTN_MARGINS")
    if not path:
        return
    import parity_util
    if parity_util.MARGINS:
        with open(path, "w") as fh:
            json.dump(parity_util.MARGINS, fh, indent=0)
