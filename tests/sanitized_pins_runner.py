"""Runs every oracle pin against the sanitizer build named on the command
line (started by test_oracle_sanitized.py with the ASan runtime preloaded):
exit status 0 if all pins pass; a sanitizer report aborts the process."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import pins  # noqa: E402


def main() -> int:
    orc = oracle.Oracle(sys.argv[1])
    failed = []
    for name in sorted(pins.ALL_PINS):
        errs = pins.ALL_PINS[name](orc)
        print(f"{name}: {'ok' if not errs else errs[:3]}", flush=True)
        if errs:
            failed.append(name)
    print(f"{len(pins.ALL_PINS) - len(failed)} of {len(pins.ALL_PINS)} pins pass", flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main())
