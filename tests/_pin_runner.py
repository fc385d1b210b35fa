"""Run every oracle pin against the oracle library at argv[1]; exit 0 when
all hold, 1 when any fails (failures printed).  Used by the planted-mistake
tests, in a child process so that a planted out-of-bounds read cannot take
the test runner down."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
from tests import oracle_pins  # noqa: E402

if __name__ == "__main__":
    fails = oracle_pins.run_all(oracle.load(sys.argv[1]))
    for f in fails:
        print(f)
    sys.exit(1 if fails else 0)
