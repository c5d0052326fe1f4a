"""Run every oracle pin against a given build of kvd_oracle.c.

usage: python tests/run_pins.py LIBRARY.so
Exit status 0 when every pin holds, 1 when at least one fails.  Used by
test_oracle_mutants.py on copies of the oracle with planted mistakes.
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import oracle_pins  # noqa: E402


def main(path):
    oracle.use_library(path)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # a planted mistake may also raise other errors
            failed.append(f"{check.__name__}: {type(e).__name__}")
    print("\n".join(failed) if failed else "all pins hold", flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
