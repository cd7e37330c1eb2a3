import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter):
    try:
        from tests import margins
    except ImportError:
        return
    if not margins.RECORDS:
        return
    tr = terminalreporter
    tr.write_sep("-", "layer-output parity margins: max|gpu - oracle| / RMS(oracle), bar passed")
    for name, frac, bar, extra in margins.RECORDS:
        tr.write_line(f"{frac:9.2e}  {bar:<12} {name}{('  ' + extra) if extra else ''}")
    n_strict = sum(1 for r in margins.RECORDS if r[2] == "strict")
    tr.write_line(f"{n_strict} of {len(margins.RECORDS)} comparisons within the strict 2e-2 RMS bar; "
                  "the rest within it plus half a bf16 ulp of each reference element")
