"""Run every oracle pin against one compiled oracle library; print the failures as JSON.

Used by test_oracle_mutants.py in a child process, so that a mutant that
crashes cannot take the test runner down with it.
"""
import json
import sys

import oracle
from tests import pins


def main(path):
    orc = oracle.Oracle(path)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, ValueError):
            failed.append(pin.__name__)
    print(json.dumps(failed))


if __name__ == "__main__":
    main(sys.argv[1])
