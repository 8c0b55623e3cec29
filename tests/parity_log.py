"""Per-case near-tie accounting of the GPU parity tests.

Every comparison of the HIP path with the oracle records, for its case, how many requests
it compared (n), how many lie in the 1e-6 near-tie band of the oracle's decision trace
(near), how many of those differ (near_mismatch) and how many differ outside it
(mismatch, which fails the test).  conftest.py prints the table at the end of the run,
so it survives `pytest -q`; with SPEC_PARITY_LOG=<path> it is also written there as JSON
lines.
"""
from __future__ import annotations

import json
import os

RECORDS: list = []


def record(label: str, stats: dict) -> None:
    rec = dict(case=label, **stats)
    RECORDS.append(rec)
    path = os.environ.get("SPEC_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def summary_lines() -> list:
    if not RECORDS:
        return []
    tot = {k: sum(r[k] for r in RECORDS) for k in ("n", "near", "near_mismatch", "mismatch")}
    lines = [f"{'case':58s} {'n':>6s} {'near':>5s} {'near_mismatch':>13s} {'mismatch':>8s}"]
    for r in RECORDS:
        lines.append(f"{r['case'][:58]:58s} {r['n']:6d} {r['near']:5d} {r['near_mismatch']:13d} "
                     f"{r['mismatch']:8d}")
    lines.append(f"{'total over ' + str(len(RECORDS)) + ' comparisons':58s} {tot['n']:6d} "
                 f"{tot['near']:5d} {tot['near_mismatch']:13d} {tot['mismatch']:8d}")
    return lines
