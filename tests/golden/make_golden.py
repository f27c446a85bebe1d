"""Writes tests/golden/oracle_tiny.json: oracle outputs on two tiny seeded cases.

The stored values come only from ``oracle/`` applied to ``make_inputs`` arrays;
the test that reads them guards the oracle against accidental changes.  Rerun
only when a change to the oracle's arithmetic is justified by the pages (and say
which passage in the commit message).
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import mhc_oracle as O  # noqa: E402
from residual_stream_amd.inputs import make_inputs  # noqa: E402

CASES = [dict(T=2, N=2, D=4, seed=31, alpha=1.0), dict(T=2, N=4, D=8, seed=32, alpha=0.5)]


def compute(case):
    inp = make_inputs(case["T"], case["N"], case["D"], seed=case["seed"], alpha=case["alpha"],
                      grads=True)
    pre = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
    xn = O.hc_post(inp.x, inp.y, pre["H_post"], pre["H_res"])
    dx, dy, dHp, dHr = O.hc_post_bwd(inp.dx_next, inp.x, inp.y, pre["H_post"], pre["H_res"])
    g = O.hc_pre_bwd(inp.dh, inp.x, inp.phi, inp.bias, dHp, dHr, inp.alphas, inp.eps, inp.iters)
    out = {"h": pre["h"], "H_pre": pre["H_pre"], "H_post": pre["H_post"], "H_res": pre["H_res"],
           "x_next": xn, "dx": dx + g["dx"], "dy": dy, "dphi": g["dphi"], "dbias": g["dbias"],
           "dalpha": g["dalpha"]}
    return {k: v.ravel().tolist() for k, v in out.items()}


def main():
    doc = {"note": "oracle outputs; written by tests/golden/make_golden.py", "cases": []}
    for case in CASES:
        doc["cases"].append({"case": case, "expected": compute(case)})
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
