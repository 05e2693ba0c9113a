"""Measured parity errors of the GPU tests, one JSON line per checked case.

When the environment variable PARITY_LOG names a file, every GPU parity check
appends {"case": ..., "tol": ..., "errors": {output: max-norm relative error}}
to it, so the margins to the tolerances are on record (pytest -q hides the
printed lines).  Without PARITY_LOG nothing is written.
"""
import json
import os


def record(case: str, tol: float, errs: dict) -> None:
    path = os.environ.get("PARITY_LOG")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps({"case": case, "tol": tol, "errors": {k: float(v) for k, v in errs.items()}}) + "\n")
