"""Write ``oracle_tiny.json``: a small oracle input/output pair.

It calls only the oracle.  The stored output is a regression fixture for the
oracle itself (it catches an accidental change to the oracle's arithmetic);
its correctness rests on the pins in ``tests/pins.py``, not on this file.
Run from the repository root: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(20261202)
    b, L, nh, p, n, g = 1, 7, 2, 3, 4, 1
    inp = dict(
        x=rng.standard_normal((b, L, nh, p)).round(3),
        dt=np.log1p(np.exp(rng.standard_normal((b, L, nh)))).round(3),
        A=(-np.exp(rng.uniform(0, np.log(16), nh))).round(3),
        B=rng.standard_normal((b, L, g, n)).round(3),
        C=rng.standard_normal((b, L, g, n)).round(3),
        D=rng.standard_normal(nh).round(3),
        h0=(0.1 * rng.standard_normal((b, nh, p, n))).round(3),
    )
    y, fin, _ = oracle.scan(**inp)
    out = {
        "citation": "Written by tests/golden/make_golden.py from oracle.scan only.",
        "inputs": {k: v.tolist() for k, v in inp.items()},
        "y": y.tolist(),
        "final": fin.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
