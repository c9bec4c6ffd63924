"""Record of how often the GPU parity tests lean on the two-phase fp64 floor.

The parity bar of the GPU tests is, per element,
    max(1e-10 |oracle|, 1e-13, FLOOR_FACTOR * B)
with B the oracle's first-order floor of the two-phase method
(oracle.hgp_rounding_bound; for integrals plus a quarter of
oracle.contraction_rounding_bound, the contraction sums' floor, so that the
bar is 4 B + C).  FLOOR_FACTOR = 4 is the factor the binary128
adjudication supports (tests/test_oracle_quad.py: the emulated fp64 method
needs at most 3.2 x B on the hardest quartets).  Every parity check appends one
JSON line to parity_floor_usage.jsonl in the results folder: the test, the check, the
number of elements, how many missed the plain 1e-10/1e-13 bar (and were
accepted only through the floor), and the largest |gpu - oracle| / B among
those.
"""
import json
import os

FLOOR_FACTOR = 4.0

_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                     "parity_floor_usage.jsonl")


def record(what: str, n_elements: int, n_plain_miss: int, max_err_over_B: float = 0.0, **extra) -> None:
    row = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "check": what,
           "elements": int(n_elements), "beyond_plain_bar": int(n_plain_miss),
           "max_err_over_B": round(float(max_err_over_B), 4)}
    row.update(extra)
    try:
        os.makedirs(os.path.dirname(_PATH), exist_ok=True)
        with open(_PATH, "a") as f:
            f.write(json.dumps(row) + "\n")
    except OSError:
        pass
