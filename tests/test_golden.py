"""The stored tie case equals exact integer/rational arithmetic, and the
current oracle still reproduces it (CPU only)."""
import json
import os

import numpy as np

import oracle
import oracle_pins

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_ties.json")


def load_golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    return {k: (np.array(v) if isinstance(v, list) else v) for k, v in g.items()}


def test_golden_is_exact():
    g = load_golden()
    X, C = g["X"].astype(np.int64), g["C"].astype(np.int64)
    lab, m1, m2 = oracle_pins._exact_assign(X, C)
    assert np.array_equal(g["labels"], lab)
    assert np.array_equal(g["d1"], m1.astype(np.float64))
    assert np.array_equal(g["d2"], m2.astype(np.float64))
    counts, means = oracle_pins._exact_update(X, lab, C.astype(np.float64))
    assert np.array_equal(g["counts"], counts)
    assert np.array_equal(g["C_next"], means)
    # the values stated by hand in make_golden.py
    assert g["labels"].tolist() == [[0, 1, 0, 1, 0, 0, 1, 1]]
    assert g["counts"].tolist() == [[4, 4, 0]]


def test_oracle_reproduces_golden():
    g = load_golden()
    labels, d1, d2 = oracle.assign(g["X"], g["C"])
    counts, C1, _ = oracle.update(g["X"], labels, g["C"])
    assert np.array_equal(labels, g["labels"]) and np.array_equal(counts, g["counts"])
    assert np.array_equal(C1, g["C_next"]) and np.array_equal(d1, g["d1"])
