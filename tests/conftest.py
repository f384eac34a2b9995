import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Print the parity errors of the full-size workloads (whole-tensor and
    worst-unit rel-L2) at the end of the run, passed or not."""
    gu = sys.modules.get("gpu_util")
    rows = getattr(gu, "PARITY", None) if gu else None
    if not rows:
        return
    terminalreporter.write_sep("-", "parity of the full-size workloads (rel-L2)")
    for label, e in rows:
        terminalreporter.write_line(
            "%-44s y %.2e  h %.2e  worst unit y %.2e  h %.2e  (tol %.0e)"
            % (label, e["y"], e["h"], e["worst_y"], e["worst_h"], e["tol"]))
