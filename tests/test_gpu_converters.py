"""Exhaustive on-GPU checks of the gfx950 conversion instructions the NVFP4
kernels rely on (run through the probe library's converter kernel), against
the exact decode of the formats (reading notes, section 2.1: E2M1 elements,
E4M3 block scales) written in the oracle:
  * E2M1 -> f16 and E2M1 -> f32 (scale 1) for every byte in every byte
    position of a 32-bit word (every code in both nibbles);
  * E4M3 -> f32 for every byte in every position (NaN codes 0x7F, 0xFF
    must decode to NaN);
  * f32 -> E2M1 (the quantizer's rounding, scale 1): round to nearest, ties
    to the even code, saturation at 6, sign copied, at every grid point,
    every midpoint, one ulp either side of each, beyond the top, tiny and
    zero values of both signs, and a random sample;
  * the packed f16 product E2M1 x E4M3 of the MFMA kernels, exact for every
    code and every finite scale."""

import os

import numpy as np
import pytest

from oracle import nvfp4_oracle as O

pytestmark = pytest.mark.gpu

try:
    from fp4_decode_gemv_amd import probe as P
    HAVE = os.path.exists(P.PROBE_LIB_PATH)
except ImportError:  # pragma: no cover
    HAVE = False


def _words_every_byte_everywhere():
    b = np.arange(256, dtype=np.uint32)
    return b | (b << 8) | (b << 16) | (b << 24)


def _same_values(got: np.ndarray, want: np.ndarray, what: str):
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), what
    bad = ~nan & (got != want)
    assert not bad.any(), (what, np.nonzero(bad)[0][:8], got[bad][:8], want[bad][:8])


def test_fp4_to_f16_every_code():
    out = P.convert(P.FP4_TO_F16, _words_every_byte_everywhere()).reshape(256, 4)
    h = out.astype(np.uint16).view(np.float16).astype(np.float64)       # low halves
    hh = (out >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    b = np.arange(256)
    for sel in range(4):
        _same_values(h[:, sel], O.E2M1_TABLE[b & 15], f"low nibble, byte {sel}")
        _same_values(hh[:, sel], O.E2M1_TABLE[b >> 4], f"high nibble, byte {sel}")


def test_fp4_to_f32_every_code():
    out = P.convert(P.FP4_TO_F32, _words_every_byte_everywhere()).reshape(256, 4, 2).view(np.float32)
    b = np.arange(256)
    for sel in range(4):
        _same_values(out[:, sel, 0].astype(np.float64), O.E2M1_TABLE[b & 15], f"low nibble, byte {sel}")
        _same_values(out[:, sel, 1].astype(np.float64), O.E2M1_TABLE[b >> 4], f"high nibble, byte {sel}")


def test_e4m3_to_f32_every_code():
    out = P.convert(P.FP8_TO_F32, _words_every_byte_everywhere()).reshape(256, 4).view(np.float32)
    for pos in range(4):
        _same_values(out[:, pos].astype(np.float64), O.E4M3_TABLE, f"byte {pos}")


def _rounding_inputs():
    g = O.E2M1_GRID
    mids = (g[:-1] + g[1:]) / 2
    pts = np.concatenate([g, mids, [6.5, 7.0, 12.0, 1e30, 2.0 ** -140, 1e-45, 0.1, 0.3, 5.9]]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    v = np.concatenate([pts, up, dn])
    v = np.concatenate([v, -v, [np.float32(0.0), np.float32(-0.0)]])
    rng = np.random.default_rng(5)
    r = (rng.standard_normal(4000) * 3).astype(np.float32)
    return np.concatenate([v, r]).astype(np.float32)


def test_f32_to_e2m1_rounding():
    v = _rounding_inputs()
    if v.size % 2:
        v = np.append(v, np.float32(1.0))
    out = P.convert(P.F32_TO_FP4, v.view(np.uint32)) & 0xFF
    want = O.e2m1_encode(v)
    got = np.empty(v.size, dtype=np.uint8)
    got[0::2] = out & 0xF
    got[1::2] = out >> 4
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (v[bad][:8], got[bad][:8], want[bad][:8])


def test_f16_block_scale_products_are_exact():
    """Every E2M1 value times every finite E4M3 value as one packed f16
    multiply equals the exact product (at most 6 significant bits, inside
    the normal f16 range)."""
    codes = np.arange(16)
    scales = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    cv = np.repeat(O.E2M1_TABLE[codes], scales.size)
    sv = np.tile(O.E4M3_TABLE[scales], codes.size)
    exact = cv * sv
    assert np.array_equal(exact.astype(np.float16).astype(np.float64), exact)  # representable
    a16 = cv.astype(np.float16).view(np.uint16).astype(np.uint32)
    s16 = sv.astype(np.float16).view(np.uint16).astype(np.uint32)
    words = np.empty(2 * cv.size, dtype=np.uint32)
    words[0::2] = a16 | (a16 << 16)
    words[1::2] = s16 | (s16 << 16)
    out = P.convert(P.F16_SCALE_MUL, words)
    lo = (out & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    hi = (out >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    _same_values(lo, exact, "low half")
    _same_values(hi, exact, "high half")
