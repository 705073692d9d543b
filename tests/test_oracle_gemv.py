"""Pins of the oracle GEMV: exact rational arithmetic on tiny inputs (decoded
through the golden E2M1 table and torch's E4M3 cast, not the oracle's own
tables), one-hot weight rows, and structural invariants."""

import json
import os
from fractions import Fraction

import numpy as np
import torch

from conftest import GOLDEN
from oracle import nvfp4_oracle as O


def _tables():
    with open(os.path.join(GOLDEN, "e2m1_codes.json")) as f:
        g = json.load(f)
    e2m1 = [Fraction(g["codes"][str(c)]) for c in range(16)]
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    e4m3 = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return e2m1, e4m3


def _rand_q(rng, rows, K):
    codes = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    scales = rng.choice(finite, (rows, K // 16)).astype(np.uint8)
    gs = np.float32(rng.uniform(1e-3, 10.0))
    return codes, scales, gs


def _exact(q, e2m1, e4m3):
    codes, scales, gs = q
    rows = codes.shape[0]
    K = codes.shape[1] * 2
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            byte = int(codes[r, k // 2])
            c = (byte & 0x0F) if k % 2 == 0 else (byte >> 4)
            row.append(e2m1[c] * Fraction(float(e4m3[scales[r, k // 16]])) * Fraction(float(gs)))
        out.append(row)
    return out


def test_gemv_matches_exact_rationals_on_tiny_inputs():
    e2m1, e4m3 = _tables()
    rng = np.random.default_rng(21)
    for M, N, K in [(1, 1, 16), (2, 3, 32), (8, 4, 64), (5, 2, 48)]:
        a = _rand_q(rng, M, K)
        w = _rand_q(rng, N, K)
        y, ref_abs = O.gemv_ref(a, w)
        A = _exact(a, e2m1, e4m3)
        W = _exact(w, e2m1, e4m3)
        for m in range(M):
            for n in range(N):
                ex = sum(A[m][k] * W[n][k] for k in range(K))
                ab = sum(abs(A[m][k] * W[n][k]) for k in range(K))
                assert abs(Fraction(y[m, n]) - ex) <= Fraction(1, 10 ** 14) * ab
                assert abs(Fraction(ref_abs[m, n]) - ab) <= Fraction(1, 10 ** 14) * ab


def test_one_hot_weight_rows_reproduce_the_activation():
    e2m1, e4m3 = _tables()
    rng = np.random.default_rng(22)
    M, K = 4, 64
    a = _rand_q(rng, M, K)
    N = K
    wc = np.zeros((N, K // 2), np.uint8)
    for n in range(N):                       # row n has 1.0 at column n
        wc[n, n // 2] = 0x02 if n % 2 == 0 else 0x20
    ws = np.full((N, K // 16), 0x38, np.uint8)   # E4M3 1.0
    y, _ = O.gemv_ref(a, (wc, ws, np.float32(1.0)))
    A = _exact(a, e2m1, e4m3)
    for m in range(M):
        for k in range(K):
            assert Fraction(y[m, k]) == A[m][k]


def test_row_permutation_commutes_and_ref_abs_bounds():
    rng = np.random.default_rng(23)
    a = _rand_q(rng, 3, 128)
    w = _rand_q(rng, 10, 128)
    y, ra = O.gemv_ref(a, w)
    p = rng.permutation(10)
    y2, ra2 = O.gemv_ref(a, (w[0][p], w[1][p], w[2]))
    # BLAS may block the sums differently; agree far below the 1e-5 tolerance
    assert np.all(np.abs(y2 - y[:, p]) <= 1e-13 * ra[:, p])
    assert np.all(np.abs(ra2 - ra[:, p]) <= 1e-13 * ra[:, p])
    assert np.all(ra >= np.abs(y))


def test_per_token_global_scales_match_exact_rationals():
    """One activation global scale per row: y[m] uses row m's own scale
    (exact rationals, each row decoded with its own scale)."""
    e2m1, e4m3 = _tables()
    rng = np.random.default_rng(23)
    M, N, K = 3, 2, 32
    codes, scales, _ = _rand_q(rng, M, K)
    gs = np.array([0.25, 3.0, 1e-3], np.float32)
    w = _rand_q(rng, N, K)
    y, ref_abs = O.gemv_ref((codes, scales, gs), w)
    W = _exact(w, e2m1, e4m3)
    for m in range(M):
        A = _exact((codes[m:m + 1], scales[m:m + 1], gs[m]), e2m1, e4m3)[0]
        for n in range(N):
            ex = sum(A[k] * W[n][k] for k in range(K))
            ab = sum(abs(A[k] * W[n][k]) for k in range(K))
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(1, 10 ** 14) * ab
            assert abs(Fraction(ref_abs[m, n]) - ab) <= Fraction(1, 10 ** 14) * ab
