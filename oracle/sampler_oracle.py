"""CPU oracle for the decode sampler: temperature-scaled top-p (nucleus)
sampling of one token per sequence from the LM-head logits.

TEST INFRASTRUCTURE ONLY (see ``oracle/nvfp4_oracle.py`` for who may import
it).  Everything here is float64 and uses a full sort: the plain definition,
not a fast one.

Sources:

* The decode loop samples with top-p = 0.95 at the temperature the ReSET rule
  chose for the token (ReSET reading notes, section 6.1 "setup", and section
  4.3 for the temperatures; section 6.3, Table 5, sweeps top-p at a fixed
  temperature).
* Top-p sampling itself is nucleus sampling as published by Holtzman et al.
  ("The Curious Case of Neural Text Degeneration", ICLR 2020): keep the
  smallest set of most probable tokens whose probability mass reaches p,
  renormalise it and draw from it.

Readings taken where the pages are silent (listed in the design notes):

* probabilities are softmax(z / T) over all N logits, with T > 0;
* "most probable first" is the order of decreasing logit, equal logits in
  increasing token index (so the order is exact and never depends on how a
  probability was rounded);
* the nucleus is the shortest prefix of that order whose cumulative mass is
  >= top_p (at least the top token; all N when top_p = 1);
* the draw uses one uniform number u in [0, 1) per sequence, passed in by the
  caller: the sampled token is the first one in the nucleus whose cumulative
  mass exceeds u times the nucleus mass (inverse-CDF sampling of the
  renormalised nucleus).
"""

from __future__ import annotations

import numpy as np


def nucleus_order(logits) -> np.ndarray:
    """Token indices in sampling order: decreasing logit, ties by index."""
    z = np.asarray(logits, dtype=np.float64)
    return np.lexsort((np.arange(z.size), -z))


def sorted_cumulative(logits, T: float):
    """(order, c): the sampling order and the normalised cumulative
    probability c[k] of its first k + 1 tokens, in float64."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    s = (z - np.max(z)) / float(np.float32(T))
    e = np.exp(s)
    order = nucleus_order(z)
    c = np.cumsum(e[order]) / np.sum(e)
    return order, c


def sample_top_p(logits, T: float, top_p: float, u: float):
    """One draw: returns (token index, nucleus size)."""
    if not (T > 0):
        raise ValueError("temperature must be positive")
    if not (0.0 < top_p <= 1.0):
        raise ValueError("top_p must be in (0, 1]")
    order, c = sorted_cumulative(logits, T)
    n = min(int(np.searchsorted(c, top_p, side="left")) + 1, c.size)  # first k with c[k] >= top_p
    r = float(u) * c[n - 1]
    j = int(np.searchsorted(c[:n], r, side="right"))                   # first k with c[k] > r
    return int(order[j]), n


def sample_rows(logits, T, top_p: float, u):
    """Row-wise draws for a [M][N] logit matrix with temperatures T [M] and
    uniforms u [M]: (tokens [M], nucleus sizes [M])."""
    L = np.asarray(logits)
    out = [sample_top_p(L[m], float(T[m]), top_p, float(u[m])) for m in range(L.shape[0])]
    return np.array([o[0] for o in out], dtype=np.int64), np.array([o[1] for o in out], dtype=np.int64)
