"""Writes tests/golden/oracle_small.json from the CPU oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
The inputs are drawn by the shared seeded generator; every stored value comes
from oracle.attention_forward.  The fixture guards against unintended changes
to the oracle's arithmetic.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

CASES = [
    dict(B=1, H_q=2, H_kv=1, N=5, D=4, causal=True, sm_scale=0.5, seed=1001),
    dict(B=1, H_q=2, H_kv=2, N=6, D=3, causal=False, sm_scale=0.577, seed=1002),
]


def main():
    out = {"about": "oracle output on tiny seeded bf16 inputs (see make_golden.py)", "cases": []}
    for c in CASES:
        q, k, v = (workloads.to_float64(t) for t in workloads.make_inputs(
            c["B"], c["H_q"], c["H_kv"], c["N"], c["D"], c["seed"]))
        O, L = oracle.attention_forward(q, k, v, is_causal=c["causal"], sm_scale=c["sm_scale"])
        out["cases"].append(dict(c, O=[float(x) for x in O.ravel()],
                                 LSE=[float(x) for x in L.ravel()]))
    with open(os.path.join(ROOT, "tests", "golden", "oracle_small.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
