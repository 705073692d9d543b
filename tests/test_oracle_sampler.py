"""Pins of the top-p sampler oracle: hand-worked draws (tests/golden), closed
forms for equal logits, the greedy limit, and the distribution of draws over
a fine grid of u against softmax probabilities computed independently."""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

from conftest import GOLDEN
from oracle import sampler_oracle as S


def _cases():
    with open(os.path.join(GOLDEN, "top_p_hand_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_draws(case):
    z = np.array(case["logits"], dtype=np.float32)
    for u, tok in zip(case["u"], case["tokens"]):
        t, n = S.sample_top_p(z, case["T"], case["top_p"], u)
        assert (t, n) == (tok, case["nucleus"]), (case["name"], u, t, n)


@pytest.mark.parametrize("N,top_p", [(7, 0.5), (100, 0.95), (151936, 0.95), (1000, 0.333)])
def test_equal_logits_closed_form(N, top_p):
    """Equal logits: the nucleus is the first ceil(top_p N) tokens in index
    order and the draw is token floor(u n) (u kept off the cell edges)."""
    z = np.full(N, -1.25, dtype=np.float32)
    n = math.ceil(top_p * N)
    for u in (0.0, 0.3141, 0.5, 0.9999):
        k = u * n
        if abs(k - round(k)) < 1e-6 and k != 0:
            continue
        t, nn = S.sample_top_p(z, 0.8, top_p, u)
        assert nn == n and t == int(math.floor(k)), (N, top_p, u, t, nn)


def test_greedy_limit():
    rng = np.random.default_rng(5)
    for _ in range(20):
        z = rng.standard_normal(300).astype(np.float32) * 3
        z[rng.integers(0, 300, 3)] = z.max()          # tied maxima: the lowest index wins
        for u in (0.0, 0.5, 0.999):
            t, n = S.sample_top_p(z, 0.6, 1e-9, u)
            assert n == 1 and t == int(np.argmax(z))


def test_draw_distribution_matches_renormalised_nucleus():
    """Draws over u = (k + 1/2) / G hit each nucleus token with frequency
    p_i / (nucleus mass) within 1/G per cell edge, and the nucleus is the
    minimal set of most probable tokens reaching top_p."""
    rng = np.random.default_rng(11)
    G = 20000
    for trial in range(6):
        N = int(rng.integers(20, 80))
        z = (rng.standard_normal(N) * rng.uniform(0.5, 3.0)).astype(np.float32)
        T = float(np.float32(rng.uniform(0.3, 1.5)))
        top_p = float(rng.uniform(0.5, 0.99))
        p = softmax(z.astype(np.float64) / T)
        counts = np.zeros(N)
        sizes = set()
        for k in range(G):
            t, n = S.sample_top_p(z, T, top_p, (k + 0.5) / G)
            counts[t] += 1
            sizes.add(n)
        assert len(sizes) == 1
        drawn = counts > 0
        mass = p[drawn].sum()
        assert mass >= top_p - 1e-12                                # reaches top_p
        assert mass - p[drawn].min() < top_p                        # minimal
        assert p[drawn].min() >= p[~drawn].max(initial=0.0)         # the most probable ones
        assert np.all(np.abs(counts[drawn] / G - p[drawn] / mass) <= 2.0 / G)


def test_row_helper_and_argument_checks():
    z = np.array([[0.0, 1.0, 2.0], [2.0, 1.0, 0.0]], dtype=np.float32)
    t, n = S.sample_rows(z, [1.0, 1.0], 1e-6, [0.5, 0.5])
    assert list(t) == [2, 0] and list(n) == [1, 1]
    with pytest.raises(ValueError):
        S.sample_top_p(z[0], 0.0, 0.9, 0.5)
    with pytest.raises(ValueError):
        S.sample_top_p(z[0], 1.0, 1.5, 0.5)
