"""Write tests/golden/wkv_exact_cases.json from oracle/exact.py only.

Each case is one channel with rational exponentials: d = e^{-w}, U = e^{u},
E_i = e^{k_i}.  Expected y and gradients are exact rationals of the weighted
sum in "RWKV（Receptance Weighted Key Value）概念", section 3.2.

Case "hand" can be checked by hand: d = 1/2, U = 1, E = (1, 1, 1), v = (1, 2, 3):
  y_1 = v_1 = 1
  y_2 = (1*1 + 1*2) / (1 + 1) = 3/2
  y_3 = (1/2*1 + 1*2 + 1*3) / (1/2 + 1 + 1) = (11/2) / (5/2) = 11/5

Run:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys
from fractions import Fraction as F

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))

from oracle.exact import loss_grads_exact  # noqa: E402

CASES = [
    dict(name="hand", d=F(1, 2), U=F(1), E=[F(1), F(1), F(1)], v=[F(1), F(2), F(3)],
         gy=[F(1), F(1), F(1)]),
    dict(name="mixed", d=F(3, 4), U=F(2), E=[F(1), F(4), F(1, 2), F(8), F(1)],
         v=[F(1), F(-2), F(3), F(0), F(5, 2)], gy=[F(1), F(-1), F(2), F(1, 2), F(3)]),
    dict(name="fast_decay", d=F(1, 8), U=F(1, 4), E=[F(2), F(1, 16), F(32), F(1), F(1, 2), F(4)],
         v=[F(-1), F(3), F(1, 3), F(2), F(-5), F(1)], gy=[F(2), F(1), F(-1), F(1), F(1, 3), F(-2)]),
    dict(name="slow_decay", d=F(255, 256), U=F(3), E=[F(1, 4), F(1), F(2), F(1, 2), F(1), F(8), F(1, 8)],
         v=[F(2), F(-1), F(1, 2), F(4), F(-3), F(1), F(0)], gy=[F(1), F(2), F(-1), F(1, 2), F(1), F(-1), F(3)]),
]


def s(x: F) -> str:
    return f"{x.numerator}/{x.denominator}"


def main() -> None:
    out = {
        "source": "RWKV（Receptance Weighted Key Value）概念, section 3.2, weighted-sum definition of wkv_t",
        "generator": "tests/golden/make_golden.py via oracle/exact.py (exact rational arithmetic)",
        "convention": "d = e^{-w}, U = e^{u}, E_i = e^{k_i}; L = sum_t gy_t y_t; dw is dL/dw",
        "cases": [],
    }
    for c in CASES:
        y, dk, dv, dw, du = loss_grads_exact(c["d"], c["U"], c["E"], c["v"], c["gy"])
        out["cases"].append({
            "name": c["name"],
            "d": s(c["d"]), "U": s(c["U"]),
            "E": [s(x) for x in c["E"]], "v": [s(x) for x in c["v"]], "gy": [s(x) for x in c["gy"]],
            "y": [s(x) for x in y], "dk": [s(x) for x in dk], "dv": [s(x) for x in dv],
            "dw": s(dw), "du": s(du),
        })
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "wkv_exact_cases.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, ensure_ascii=False)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
