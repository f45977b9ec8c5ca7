"""Write tests/golden/tiny_ties.json.  Calls only the oracle.

The case is small enough to check by hand: d = 2, N = 8, K = 3, integer
coordinates, centroid 2 duplicates centroid 0 (every point is exactly as far
from both) and several points sit exactly midway between centroids 0 and 1.
The pages fix no tie rule; the reading used is that the lowest index wins.
Expected by hand: labels 0 1 0 1 0 0 1 1; counts 4 4 0; centroid 0 = (1/4, 1/4),
centroid 1 = (3, 5/4), centroid 2 (empty) keeps (0, 0).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402

X = np.array([[[1, 0], [2, 1], [-1, -1], [3, 0], [0, 1], [1, 1], [2, -1], [5, 5]]], np.float64)
C = np.array([[[0, 0], [2, 0], [0, 0]]], np.float64)


def main():
    labels, d1, d2 = oracle.assign(X, C)
    counts, C1, bad = oracle.update(X, labels, C)
    assert bad == 0
    out = {
        "source": "hand-checkable tie case; values written by tests/golden/make_golden.py "
                  "(oracle only)",
        "X": X.tolist(), "C": C.tolist(),
        "labels": labels.tolist(), "d1": d1.tolist(), "d2": d2.tolist(),
        "counts": counts.tolist(), "C_next": C1.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_ties.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
