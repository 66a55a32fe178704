import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """With MFIN_ACCURACY_JSON set, the GPU parity tests' accuracy records (one per configuration
    sub-case: max ulp, counts, mean |err| against FP64 beside the rounding floor) go to that
    file."""
    path = os.environ.get("MFIN_ACCURACY_JSON")
    if not path:
        return
    from tests import parity
    if parity.ACCURACY:
        parity.write_accuracy(path, "MFIN_ACCURACY_JSON=" + path + " python -m pytest "
                              + " ".join(session.config.invocation_params.args))
