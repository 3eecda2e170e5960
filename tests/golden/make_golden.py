"""Writes worked_example.json: a tiny diagonal-model case with dyadic-rational
inputs and its EXACT filtering outputs, computed by oracle.gaussian (exact
joint-Gaussian marginalisation over Fractions, no recursion).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction as Fr

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle.gaussian import diag_forward_exact  # noqa: E402

# B=1, H=1, T=3, dk=2, dv=2.  Dyadic rationals are exact in binary floating point.
q = [[Fr(1), Fr(1, 2)], [Fr(-1, 2), Fr(3, 4)], [Fr(1, 4), Fr(-1)]]
k = [[Fr(1), Fr(-1, 2)], [Fr(3, 4), Fr(1, 4)], [Fr(-1, 2), Fr(1)]]
v = [[Fr(1), Fr(-2)], [Fr(1, 2), Fr(3, 2)], [Fr(-1, 4), Fr(1)]]
a = [[Fr(1, 2), Fr(7, 8)], [Fr(3, 4), Fr(1, 2)], [Fr(7, 8), Fr(3, 4)]]
qn = [Fr(1, 4), Fr(1, 8)]
r = [Fr(1, 2), Fr(1), Fr(2)]
l0 = [Fr(1), Fr(2)]
eta0 = [[Fr(1, 2), Fr(0)], [Fr(-1, 4), Fr(1)]]

o, l_hist, etaT = diag_forward_exact(q, k, v, a, qn, r, l0, eta0)


def enc(x):
    if isinstance(x, list):
        return [enc(y) for y in x]
    return str(x)


doc = {
    "what": "diagonal KLA filter, B=1 H=1 T=3 dk=2 dv=2, exact rational outputs",
    "source": "oracle/gaussian.py (joint-Gaussian marginalisation, Fractions)",
    "inputs": {"q": enc(q), "k": enc(k), "v": enc(v), "a": enc(a), "qn": enc(qn),
               "r": enc(r), "l0": enc(l0), "eta0": enc(eta0)},
    "outputs": {"o": enc(o), "l_all": enc(l_hist), "etaT": enc(etaT)},
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_example.json"), "w") as f:
    json.dump(doc, f, indent=1)
print("o[2] =", [float(x) for x in o[2]])
