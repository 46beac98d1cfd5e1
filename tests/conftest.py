import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (HERE, ROOT):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running GPU parity case")


@pytest.fixture(scope="session")
def oracle_run():
    import oracle
    return oracle.run


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on the real stderr before it touches the GPU, so a run that
    ends abruptly still shows which case was running."""
    if request.node.get_closest_marker("gpu"):
        sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield


def pytest_sessionfinish(session, exitstatus):
    """With GDN_PARITY_REPORT=<path>, write the full-size error summary the parity tests
    recorded (tests/parity.py) to that path."""
    path = os.environ.get("GDN_PARITY_REPORT")
    if not path:
        return
    import parity
    if parity.REPORT:
        cmd = "GDN_PARITY_REPORT=" + path + " python -m pytest " + " ".join(session.config.args)
        parity.write_report(path, "Command (repo root, MI355X): `" + cmd + " -m gpu`. Every "
                            "row is one workload and method; errors are per V head (output "
                            "max|err| over the head's outputs divided by their RMS; state "
                            "Frobenius error over the head's state divided by its norm), "
                            "worst over what was compared. Session exit status: "
                            + str(int(exitstatus)) + ".")
