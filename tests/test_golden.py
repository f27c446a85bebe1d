"""The oracle still reproduces the stored tiny-case outputs (regression guard)."""

import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_reproduces_golden():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        doc = json.load(f)
    assert len(doc["cases"]) == len(mg.CASES)
    for entry in doc["cases"]:
        now = mg.compute(entry["case"])
        for k, v in entry["expected"].items():
            np.testing.assert_allclose(now[k], v, rtol=1e-12, atol=1e-14, err_msg=k)
