"""Pins of the entropy and ReSET oracle: closed-form entropies and hand-worked
temperature sequences (tests/golden), plus invariants."""

import json
import math
import os

import numpy as np

from conftest import GOLDEN
from oracle import reset_oracle as R


def _g(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_entropy_closed_forms():
    g = _g("entropy_closed_forms.json")
    N = g["N"]
    z = np.zeros(N)
    assert abs(R.entropy(z) - g["uniform"]) < 1e-12
    z1 = z.copy(); z1[123] = 20.0
    assert abs(R.entropy(z1) - g["one_at_20"]) < 1e-12
    z8 = z.copy(); z8[[1, 5, 99, 1000, 5000, 70000, 100000, 151935]] = 10.0
    assert abs(R.entropy(z8) - g["eight_at_10"]) < 1e-11
    assert abs(g["uniform"] - math.log(N)) < 1e-15


def test_entropy_invariants():
    rng = np.random.default_rng(31)
    z = rng.standard_normal(5000) * 2
    h = R.entropy(z)
    assert abs(R.entropy(z + 123.0) - h) < 1e-12          # shift invariance
    assert abs(R.entropy(rng.permutation(z)) - h) < 1e-12  # permutation invariance
    assert 0 <= h <= math.log(5000)
    assert R.entropy(z * 1e4) < 1e-6                      # near one-hot


def test_hand_worked_sequences():
    for seq in _g("reset_hand_sequences.json")["sequences"]:
        p = R.ResetParams(**seq["params"])
        tr = R.reset_sequence(seq["H"], seq["step_start"], p)
        assert np.allclose(tr.T, seq["T"], atol=0), seq["name"]
        if seq["uncertain"] is not None:
            assert list(tr.uncertain) == seq["uncertain"], seq["name"]


def test_constant_entropy_is_never_uncertain():
    # dyadic values keep every mean exact, so Hstep == Hbar exactly
    p = R.ResetParams(window=4)
    for h in (0.25, 0.5, 3.0):
        flags = np.zeros(40, np.uint8); flags[[0, 7, 21]] = 1
        tr = R.reset_sequence(np.full(40, h), flags, p)
        assert not tr.uncertain.any()
        assert np.all(tr.T == (p.t_low if h < p.tau0 else p.t_high))


def test_batch_columns_are_independent():
    rng = np.random.default_rng(32)
    H = rng.uniform(0, 3, (50, 3))
    f = (rng.random((50, 3)) < 0.1).astype(np.uint8); f[0] = 1
    p = R.ResetParams()
    b = R.reset_batch(H, f, p)
    for m in range(3):
        assert np.array_equal(b[m].T, R.reset_sequence(H[:, m], f[:, m], p).T)
