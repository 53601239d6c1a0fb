import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle work")


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library through its Python binding (loads or raises)."""
    import moe_decoder_step_amd as m
    m.load()
    return m


def pytest_terminal_summary(terminalreporter):
    """The achieved error of every float comparison of the run, by test: the
    worst elementwise max|d|/max(1,|ref|) and max|d|/max|ref| against the
    tolerance."""
    from tests._util import ACHIEVED
    if not ACHIEVED:
        return
    worst = {}
    for test, what, rel, nrm, tol in ACHIEVED:
        w = worst.get(test)
        if w is None or nrm / tol > w[2] / w[3]:
            worst[test] = (what, rel, nrm, tol)
    tr = terminalreporter
    tr.section("achieved float error (worst comparison per test)")
    for test, (what, rel, nrm, tol) in sorted(worst.items()):
        tr.write_line(f"{rel:9.2e} {nrm:9.2e}  tol {tol:.0e}  {test}  [{what}]")
    allw = max(ACHIEVED, key=lambda a: a[3] / a[4])
    tr.write_line(f"{len(ACHIEVED)} comparisons; worst max|d|/max|ref| = {allw[3]:.2e} "
                  f"({allw[3] / allw[4]:.1%} of its tolerance) in {allw[0]} [{allw[1]}]")
