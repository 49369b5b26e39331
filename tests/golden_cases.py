"""Reader for the fixtures in tests/golden/: builds input rows and expected rows."""
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name="closed_forms.json"):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)["cases"]


def row(spec, cols, dtype=np.float64):
    """A row of `cols` values from a fixture spec (fill / head / at, rest 0)."""
    out = np.full(cols, float(spec.get("fill", spec.get("rest", 0.0))), dtype=dtype)
    if "head" in spec:
        out[: len(spec["head"])] = spec["head"]
    for idx, val in spec.get("at", []):
        out[idx] = val
    return out


def expected(spec, cols):
    if "all" in spec:
        return np.full(cols, float(spec["all"]))
    return row({k: v for k, v in spec.items() if k in ("head", "at", "rest")}, cols)
