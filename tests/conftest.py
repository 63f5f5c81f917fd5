import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """Write every parity comparison's errors (tests/_gpu.py RECORD) to the file
    named by PKV_PARITY_RECORD, with the command that produced them."""
    import json

    path = os.environ.get("PKV_PARITY_RECORD")
    if not path or "tests._gpu" not in sys.modules:
        return
    rec = sys.modules["tests._gpu"].RECORD
    if not rec:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"command": " ".join(sys.argv), "exit_status": int(exitstatus), "comparisons": rec}, f,
                  indent=1)
        f.write("\n")
