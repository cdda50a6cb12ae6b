import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def c_oracle():
    from oracle import c_oracle as co
    co.build(force=False)
    return co


def pytest_terminal_summary(terminalreporter):
    """Max- and mean-abs error of every full-workload parity comparison."""
    try:
        from tests._helpers import PARITY_LOG
    except Exception:
        return
    if not PARITY_LOG:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity against the fp64 oracle (full workloads)")
    for what, dt, n, mx, mean in PARITY_LOG:
        tr.write_line(f"{what:<44s} {dt:<5s} {n:>10d} elems  max-abs {mx:.3e}  mean-abs {mean:.3e}")
    path = os.environ.get("PKV_PARITY_LOG")
    if path:
        import json
        with open(path, "w") as f:
            json.dump([dict(what=w, kv_dtype=d, elems=n, max_abs=mx, mean_abs=me) for w, d, n, mx, me in PARITY_LOG],
                      f, indent=1)
