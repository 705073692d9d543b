"""CPU oracle for the LM-head epilogue: token entropy and the ReSET
step-aware temperature choice.

TEST INFRASTRUCTURE ONLY (see ``oracle/nvfp4_oracle.py`` for who may import
it).  Everything here is float64 and recomputes every mean from the full
history, so it is O(t^2) on purpose: the plain definition, not a fast one.

Sources:

* Token entropy H_t of the next-token distribution (ReSET project page,
  "Step-aware temperature scaling"; reading notes, section 3.1).
* SAT, the step-aware threshold (reading notes, section 4.1): compare the
  global running mean of token entropy with the online step-entropy
  estimate; a confident step falls back to the fixed threshold tau0, an
  uncertain step uses the step estimate itself as the threshold.
* HSE, the online step-entropy estimator (reading notes, section 4.2): the
  running mean inside the current step, except that the first w positions of
  a step use a sliding window over the last w tokens.
* Two temperatures (project page rule; reading notes, section 4.3): T_low
  when H_t is below the threshold, T_high otherwise; T_base is the model
  default and is used only when ReSET is switched off.
* The fixed-threshold rule (reading notes, section 3.1, formula (1)): the
  same two temperatures with the threshold held at tau0 for every token,
  the token-level baseline that SAT replaces.

Readings taken where the pages are silent or garbled (listed in the design
notes): natural log, softmax at temperature 1 over all logits; update first,
then decide (H_t itself enters every mean at position t); the window holds
the last min(w, t+1) entropies and crosses step boundaries; "first w
positions" means step length <= w; "uncertain" is a strict
``Hstep > Hbar``; T_low is chosen on a strict ``H_t < tau_t``.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def entropy(logits: np.ndarray) -> float:
    """H = -sum_i p_i ln p_i with p = softmax(z), in float64."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - np.max(z)
    e = np.exp(z)
    p = e / np.sum(e)
    nz = p > 0
    return float(-np.sum(p[nz] * np.log(p[nz])))


def entropy_rows(logits: np.ndarray) -> np.ndarray:
    """Entropy of each row of a [M][N] logit matrix."""
    return np.array([entropy(r) for r in np.asarray(logits)], dtype=np.float64)


@dataclass(frozen=True)
class ResetParams:
    tau0: float = 0.6
    t_low: float = 0.4
    t_high: float = 1.0
    t_base: float = 0.6
    window: int = 8
    mode: int = 0          # 0 = ReSET, 1 = BASE (always t_base), 2 = fixed threshold tau0


@dataclass
class ResetTrace:
    """Per-position intermediates of one sequence (all float64)."""

    H: np.ndarray
    Hbar: np.ndarray
    Hstep: np.ndarray
    tau: np.ndarray
    uncertain: np.ndarray
    T: np.ndarray


def reset_sequence(H, step_start, p: ResetParams) -> ResetTrace:
    """Temperatures of one sequence from its entropies H[0..P-1] and step
    flags step_start[0..P-1] (1 = this position begins a new step; position 0
    always begins one)."""
    H = np.asarray(H, dtype=np.float64)
    flags = np.asarray(step_start).astype(bool)
    P = len(H)
    Hbar = np.zeros(P)
    Hstep = np.zeros(P)
    tau = np.zeros(P)
    unc = np.zeros(P, dtype=bool)
    T = np.zeros(P)
    for t in range(P):
        hist = H[: t + 1]
        Hbar[t] = np.mean(hist)
        # first position of the step that contains t
        s0 = max(s for s in range(t + 1) if s == 0 or flags[s])
        step_len = t - s0 + 1
        in_step = np.mean(H[s0: t + 1])
        win = np.mean(H[max(0, t + 1 - p.window): t + 1])
        Hstep[t] = win if step_len <= p.window else in_step
        unc[t] = Hstep[t] > Hbar[t]
        tau[t] = Hstep[t] if unc[t] else p.tau0
        if p.mode == 2:          # formula (1): the threshold is tau0 whatever the step
            tau[t] = p.tau0
        if p.mode == 1:
            T[t] = p.t_base
        else:
            T[t] = p.t_low if H[t] < tau[t] else p.t_high
    return ResetTrace(H, Hbar, Hstep, tau, unc, T)


def reset_batch(H, step_start, p: ResetParams) -> list[ResetTrace]:
    """H, step_start: [positions][M]; one independent sequence per column."""
    H = np.asarray(H, dtype=np.float64)
    f = np.asarray(step_start)
    return [reset_sequence(H[:, m], f[:, m], p) for m in range(H.shape[1])]
