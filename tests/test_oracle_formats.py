"""Pins of the oracle's E2M1 / E4M3 tables and encoders against things other
than the oracle: the format definitions (golden files), torch's float8_e4m3fn
cast (a library routine), and brute force with exact rationals."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import nvfp4_oracle as O


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_e2m1_table_is_the_value_set():
    g = _golden("e2m1_codes.json")
    for code, val in g["codes"].items():
        c = int(code)
        assert O.E2M1_TABLE[c] == val
        assert np.signbit(O.E2M1_TABLE[c]) == (c >= 8)
    mags = sorted(set(abs(v) for v in g["codes"].values()))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert O.E2M1_GRID.max() == 6.0


def test_e2m1_tie_cases():
    g = _golden("e2m1_codes.json")
    for v, code in g["rne_ties"]["cases"]:
        assert int(O.e2m1_encode(np.float32(v))) == code, v


def test_e4m3_table_matches_torch_for_all_256_codes():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    # sign of zero for 0x80
    assert np.signbit(ours[0x80])


def test_e4m3_landmarks():
    g = _golden("e4m3_landmarks.json")
    for key in ("max_finite", "min_subnormal", "min_normal", "one"):
        code, val = g[key]
        assert O.E4M3_TABLE[code] == val, key
    assert sorted(int(c) for c in np.nonzero(np.isnan(O.E4M3_TABLE))[0]) == g["nan_codes"]
    assert len(O.E4M3_GRID) == g["finite_nonnegative_count"]
    assert np.all(np.diff(O.E4M3_GRID) > 0)
    for v, code in g["rne_cases"]["cases"]:
        assert int(O.e4m3_encode(np.float64(np.float32(v)))) == code, v


def _torch_e4m3(vals_f32):
    t = torch.from_numpy(np.minimum(vals_f32, np.float32(448.0)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(7)
    # log-uniform over the whole range the block scale can take, plus tiny
    v = np.exp2(rng.uniform(-40, 9.5, 200_000)).astype(np.float32)
    grid = O.E4M3_GRID.astype(np.float32)
    mids = ((O.E4M3_GRID[:-1] + O.E4M3_GRID[1:]) / 2).astype(np.float32)
    near = np.concatenate([grid, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           np.array([0.0, 448.0, 500.0, 1e30], np.float32)])
    for arr in (v, near):
        ours = O.e4m3_encode(arr.astype(np.float64))
        ref = _torch_e4m3(arr)
        assert np.array_equal(ours, ref)


def _brute_e2m1(x: float) -> int:
    """Nearest magnitude with exact rationals; ties to the even code."""
    fx = Fraction(abs(x))
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    best = None
    for c, m in enumerate(mags):
        d = abs(fx - m)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    sign = 1 if np.signbit(np.float32(x)) else 0
    return best[1] | (sign << 3)


def test_e2m1_encode_bruteforce_over_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    # restrict to magnitudes where something happens (others saturate / flush),
    # plus a sample of the rest
    interesting = f[(np.abs(f) < 16)]
    rng = np.random.default_rng(3)
    sample = np.concatenate([interesting, rng.choice(f, 2000, replace=False)])
    for scale in (np.float32(1.0), np.float32(0.75), np.float32(3.0)):
        with np.errstate(over="ignore"):
            vals = (sample * scale).astype(np.float32)
        vals = vals[np.isfinite(vals)]
        ours = O.e2m1_encode(vals)
        ref = np.array([_brute_e2m1(float(x)) for x in vals], dtype=np.uint8)
        assert np.array_equal(ours, ref), scale


def test_e2m1_encode_at_midpoints_and_neighbours():
    mids = (O.E2M1_GRID[:-1] + O.E2M1_GRID[1:]) / 2
    pts = []
    for m in mids.astype(np.float32):
        pts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(100))]
    pts = np.array(pts + [-p for p in pts], dtype=np.float32)
    ours = O.e2m1_encode(pts)
    ref = np.array([_brute_e2m1(float(x)) for x in pts], dtype=np.uint8)
    assert np.array_equal(ours, ref)
