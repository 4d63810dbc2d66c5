"""Write the exact-rational fixtures in this folder.

Calls only the oracle's exact-rational recurrence (oracle/exact.py); the pages
print no worked example, so every stored value here is an exact rational
result of the recurrence of the OSDN technical summary (gist.science,
"OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
Attention", §1, §2.1-2.3) on small rational inputs, stored as "p/q" strings.

    python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction as Fr

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import exact  # noqa: E402


def _s(x):
    if isinstance(x, list):
        return [_s(y) for y in x]
    return str(Fr(x))


CASES = {
    # vanilla OSDN, non-unit keys, nonzero initial state and preconditioner
    "vanilla_T5_dk3_dv2": dict(
        q=[[1, 0, -1], [Fr(1, 2), 1, 0], [0, 0, 1], [1, 1, 1], [-1, Fr(1, 3), 0]],
        k=[[Fr(1, 2), Fr(1, 2), 0], [0, 1, Fr(-1, 2)], [Fr(3, 4), 0, Fr(1, 4)],
           [Fr(1, 3), Fr(-2, 3), Fr(2, 3)], [1, 0, 0]],
        v=[[1, -1], [2, 0], [0, Fr(1, 2)], [-1, 1], [Fr(3, 2), 2]],
        beta=[Fr(1, 2), Fr(3, 4), Fr(1, 4), 1, Fr(5, 8)],
        r=None, d0=[1, Fr(3, 2), Fr(1, 2)], S0=[[0, Fr(1, 4), 0], [Fr(-1, 2), 0, 1]],
        eta=Fr(2, 5)),
    # APF retention, a zero key (no preconditioner step) and a repeated key
    "apf_T6_dk2_dv2": dict(
        q=[[1, 0], [0, 1], [1, 1], [1, -1], [Fr(1, 2), 0], [0, 0]],
        k=[[Fr(3, 5), Fr(4, 5)], [0, 0], [Fr(3, 5), Fr(4, 5)], [1, 0], [0, 1], [Fr(3, 5), Fr(4, 5)]],
        v=[[1, 2], [5, 5], [1, 2], [-1, 0], [0, 3], [1, 2]],
        beta=[Fr(1, 2), Fr(1, 2), Fr(7, 8), Fr(1, 3), Fr(2, 3), 1],
        r=[Fr(9, 10), Fr(1, 2), Fr(19, 20), 1, Fr(4, 5), Fr(7, 8)],
        d0=None, S0=None, eta=Fr(1, 4)),
}


def main():
    for name, c in CASES.items():
        out = exact.run(c["q"], c["k"], c["v"], c["beta"], c["r"], c["d0"], c["S0"], c["eta"])
        rec = {"source": "oracle/exact.py (exact rational recurrence)",
               "inputs": {kk: (None if vv is None else _s(vv)) for kk, vv in c.items()},
               "outputs": {kk: _s(vv) for kk, vv in out.items()}}
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
