"""Pins of the oracle's target argmax ([TSD] "Verification and Acceptance
Algorithms": the target prediction at a node is the argmax of its logits)
against a brute-force scan written here, closed forms, and the tie and NaN
readings."""
import math

import numpy as np
import pytest

from oracle import tree_verify_oracle as O


def brute(row):
    best, bi = None, -1
    for i, v in enumerate(row):
        v = float(v)
        if bi < 0:
            best, bi = v, i
        elif math.isnan(best):
            continue
        elif math.isnan(v) or v > best:
            best, bi = v, i
    return bi


@pytest.mark.parametrize("vocab", [1, 2, 7, 64, 1000])
def test_argmax_equals_brute_force(vocab):
    rng = np.random.default_rng(vocab)
    x = rng.integers(-3, 4, (50, vocab)).astype(np.float32)   # many ties
    x[3, :] = 2.0                                           # all equal -> index 0
    if vocab > 5:
        x[5, 4] = np.nan
        x[6, 2] = np.inf
        x[6, 5] = np.nan
        x[7, :] = -np.inf
        x[8, 1] = -0.0
        x[8, :] = np.where(np.arange(vocab) == 1, -0.0, -1.0)
        x[8, 3] = 0.0                                       # -0 at 1 ties +0 at 3 -> 1
    got = O.target_argmax(x)
    assert got.tolist() == [brute(r) for r in x]
    if vocab > 5:
        assert got[3] == 0 and got[5] == 4 and got[6] == 5 and got[7] == 0 and got[8] == 1


def test_argmax_one_hot_closed_form():
    V = 151936
    idx = np.array([0, 1, V - 1, 12345, 151935 // 2])
    x = np.full((idx.size, V), -5.0, np.float32)
    x[np.arange(idx.size), idx] = 3.0
    assert O.target_argmax(x).tolist() == idx.tolist()
