import os
import sys

import pytest

ROOT = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(ROOT)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Parity reports of the GPU tests (one line per compared case), printed in the terminal summary so
# that the counts of compared requests, excused near-ties and decisions leave the test process
# even under -q.
PARITY_LINES: list = []


def record_parity(case: str, summary: str) -> None:
    PARITY_LINES.append(f"{case}: {summary}")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if PARITY_LINES:
        terminalreporter.section("parity against the fp64 oracle")
        for line in PARITY_LINES:
            terminalreporter.write_line(line)


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()
