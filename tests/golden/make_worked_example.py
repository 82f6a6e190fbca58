"""Writes worked_example.json: the pages' scalar example, solved in closed form.

Source of the inputs: FlashAttention explainer (cztcode.com/2026/5368), §2
(stable vs online softmax over four scores near 1000 with scalar values) and
§7 (the same data split into the first two and last two entries, each block
summarised and the two summaries merged).  The page prints the inputs and
asserts agreement to 1e-12 but prints no output value, so the expected values
here are the closed forms, evaluated with 50-digit decimal arithmetic:

    O   = sum_j e^(s_j - 1002) v_j / sum_j e^(s_j - 1002)
        = (2e^-2 - e^-3 + 4 + 3e^-4) / (e^-2 + e^-3 + 1 + e^-4)
    LSE = 1002 + ln(1 + e^-2 + e^-3 + e^-4)
    left  block (1000, 999):  (m, l, u) = (1000, 1 + e^-1, 2 - e^-1)
    right block (1002, 998):  (m, l, u) = (1002, 1 + e^-4, 4 + 3e^-4)
    merged: (1002, e^-2 (1 + e^-1) + 1 + e^-4, e^-2 (2 - e^-1) + 4 + 3e^-4)

This script does not touch the oracle.  Run: python tests/golden/make_worked_example.py
"""
import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 50
E = Decimal(1).exp()


def e(x):
    return Decimal(x).exp()


scores = [1000, 999, 1002, 998]
values = [2, -1, 4, 3]
m = max(scores)
w = [e(s - m) for s in scores]
den = sum(w)
num = sum(wi * vi for wi, vi in zip(w, values))
O = num / den
LSE = Decimal(m) + den.ln()

left = (1000, 1 + e(-1), 2 - e(-1))
right = (1002, 1 + e(-4), 4 + 3 * e(-4))
merged_l = e(-2) * left[1] + right[1]
merged_u = e(-2) * left[2] + right[2]

out = {
    "source": "FlashAttention explainer (cztcode.com/2026/5368), §2 and §7 scalar example",
    "scores": scores,
    "values": values,
    "O": str(O),
    "LSE": str(LSE),
    "left_state": [str(x) for x in left],
    "right_state": [str(x) for x in right],
    "merged_state": ["1002", str(merged_l), str(merged_u)],
    "merged_O": str(merged_u / merged_l),
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_example.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
    f.write("\n")
print(out["O"], out["LSE"])
