"""CPU oracle for the NVFP4 W4A4 small-M decode projection.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it and shares no code, table or constant generator with it.

What it computes, and where that comes from:

* NVFP4 format (ReSET reading notes, Paper-Reading-Collection, section 2.1
  "what format NVFP4 is", and section 6.1 "setup"): every element is a 4-bit
  E2M1 float, elements come in blocks of 16 that share one FP8 E4M3 scale, and
  the whole tensor carries one more FP32 global scale.
* The projection ``Y = X W`` at small M (ReSET project page, "Core
  contribution -- the nvfp4r CUDA-core kernel"), with the activations
  quantized on the fly to the same format (reading notes, section 5.3).

Readings taken where the pages are silent (every one is listed in the
design notes of the repository):

* global scale ``s_g = fl32(amax / 2688)`` with ``2688 = 6 * 448`` (largest
  E2M1 magnitude times largest E4M3 scale), per tensor;
* block scale ``s_b = E4M3_RNE_SAT(fl32(amax_b / fl32(6 * s_g)))``, zero when
  ``s_g == 0``;
* element ``q = E2M1_RNE_SAT(fl32(x / fl32(dec(s_b) * s_g)))`` with the sign
  bit copied from x, zero magnitude when the divisor is zero;
* RNE = round to nearest, ties to the even code; SAT = clamp to the largest
  finite magnitude (6 for E2M1, 448 for E4M3; E4M3 never produces NaN);
* two codes per byte, element 2j in the low nibble; block scales stored
  row-major ``[rows][K/16]`` (not interleaved; reading notes, section 5.3);
* dequantized value ``E2M1(q) * E4M3(s_b) * s_g``; the GEMV is the exact
  real dot product of dequantized rows, evaluated in float64.

Each floating-point step that the recipe fixes in float32 is done here in
numpy float32 (IEEE, correctly rounded); everything else is float64.
"""

from __future__ import annotations

import numpy as np

BLOCK = 16                       # elements per block scale
E2M1_MAX = 6.0
E4M3_MAX = 448.0
GLOBAL_DIVISOR = np.float32(2688.0)   # 6 * 448

# ---------------------------------------------------------------------------
# Formats: decode tables written from the bit layout of each format
# ---------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: 1 sign bit, 2 exponent bits (bias 1),
    1 mantissa bit; exponent 0 is subnormal (0 or 0.5)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 ("FN") code: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN and
    there is no infinity."""
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# non-negative finite grids, ascending; the index of a grid point is its code
E2M1_GRID = E2M1_TABLE[:8].copy()             # 0, .5, 1, 1.5, 2, 3, 4, 6
E4M3_GRID = E4M3_TABLE[:127].copy()           # 0 .. 448 (codes 0x00..0x7E)


def _nearest_even_code(grid: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to each v >= 0; a tie goes to the even
    index; values at or above the top of the grid saturate to it.

    The midpoint of two neighbouring grid points is exact in float64 (both
    are short dyadic numbers), so every comparison below is exact."""
    v = np.asarray(v, dtype=np.float64)
    top = len(grid) - 1
    lo = np.searchsorted(grid, v, side="right") - 1      # grid[lo] <= v
    lo = np.clip(lo, 0, top)
    hi = np.minimum(lo + 1, top)
    mid = (grid[lo] + grid[hi]) * 0.5
    pick_hi = (v > mid) | ((v == mid) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(v >= grid[top], top, code)
    return code.astype(np.uint8)


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """E4M3 code of each non-negative t: nearest finite value, ties to the
    even code, clamped to 448."""
    t = np.asarray(t, dtype=np.float64)
    if np.any(t < 0) or np.any(~np.isfinite(t)):
        raise ValueError("block-scale candidates must be finite and >= 0")
    return _nearest_even_code(E4M3_GRID, t)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """E2M1 code of each float: nearest magnitude in {0,.5,1,1.5,2,3,4,6},
    ties to the even code, clamped to 6; sign bit copied from v (so -0.0 and
    small negatives give code 0x8)."""
    v = np.asarray(v)
    mag = _nearest_even_code(E2M1_GRID, np.abs(v.astype(np.float64)))
    sign = np.signbit(v).astype(np.uint8)
    return (mag | (sign << 3)).astype(np.uint8)


# ---------------------------------------------------------------------------
# Quantization (the fixed recipe above)
# ---------------------------------------------------------------------------


def global_scale(amax: float) -> np.float32:
    """s_g = fl32(amax / 2688)."""
    return np.float32(np.float32(amax) / GLOBAL_DIVISOR)


def quantize_nvfp4(x: np.ndarray, gscale: float | None = None):
    """Quantize a float32 matrix [rows][K] (K % 16 == 0) to NVFP4.

    Returns ``(codes uint8 [rows][K/2], scales uint8 [rows][K/16],
    gscale float32)``.  With ``gscale=None`` the global scale comes from this
    tensor's own amax (dynamic); otherwise the given value is used (static,
    or a row subset of a larger tensor whose global scale is known)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("x must be [rows][K] with K % 16 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    rows, K = x.shape

    # step 1-2: global scale
    if gscale is None:
        amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
        s_g = global_scale(amax)
    else:
        s_g = np.float32(gscale)

    # step 3: per-block amax and block-scale candidate t_b (float32)
    xb = x.reshape(rows, K // BLOCK, BLOCK)
    amax_b = np.max(np.abs(xb), axis=2)
    if s_g == 0:
        t_b = np.zeros_like(amax_b)
    else:
        denom = np.float32(np.float32(6.0) * s_g)
        t_b = (amax_b / denom).astype(np.float32)

    # step 4: E4M3 block scale
    s_b = e4m3_encode(t_b)

    # step 5: element scale e_b = fl32(dec(s_b) * s_g), v = fl32(x / e_b)
    e_b = (E4M3_TABLE[s_b].astype(np.float32) * s_g).astype(np.float32)
    e_full = np.repeat(e_b[:, :, None], BLOCK, axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(e_full != 0, xb / np.where(e_full != 0, e_full, np.float32(1)), np.float32(0))
    v = v.astype(np.float32)
    # keep the sign of x on exact zeros (0/e and the e == 0 case)
    v = np.where(v == 0, np.copysign(np.float32(0), xb), v).astype(np.float32)

    # step 6: E2M1 codes, sign from x
    q = e2m1_encode(v).reshape(rows, K)

    # step 7: pack, element 2j in the low nibble
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, s_b.astype(np.uint8), np.float32(s_g)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 [rows][K/2] -> 4-bit codes [rows][K] (element 2j = low nibble)."""
    rows, half = codes.shape
    q = np.empty((rows, 2 * half), dtype=np.uint8)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    return q


def dequantize(codes: np.ndarray, scales: np.ndarray, gscale) -> np.ndarray:
    """Exact real values E2M1(q) * E4M3(s_b) * s_g as float64 [rows][K]
    (each product has at most 6 + 24 significant bits, exact in float64).
    ``gscale`` is one scale for the tensor, or one per row ([rows])."""
    q = unpack_codes(codes)
    vals = E2M1_TABLE[q]
    sc = np.repeat(E4M3_TABLE[scales], BLOCK, axis=1)
    g = np.asarray(gscale, dtype=np.float32).astype(np.float64)
    if g.ndim == 1:
        g = g[:, None]
    return vals * sc * g


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------


def gemv_ref(a_q, w_q):
    """y[m][n] = sum_k Ahat[m][k] * What[n][k] in float64, plus the tolerance
    reference ref_abs[m][n] = sum_k |Ahat[m][k] * What[n][k]|.

    ``a_q`` and ``w_q`` are ``(codes, scales, gscale)`` triples."""
    A = dequantize(*a_q)
    W = dequantize(*w_q)
    y = A @ W.T
    ref_abs = np.abs(A) @ np.abs(W).T
    return y, ref_abs


# ---------------------------------------------------------------------------
# Convenience for bf16 inputs
# ---------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_act_bf16(x_bits: np.ndarray, gscale: float | None = None):
    """Quantize a bf16 activation [M][K] given as bit patterns."""
    return quantize_nvfp4(bf16_to_f32(x_bits), gscale)


def quantize_act_bf16_per_token(x_bits: np.ndarray, gscales=None):
    """Per-token global scales: each row [1][K] of the bf16 activation is
    quantized as a tensor of its own (its own amax / 2688, or its entry of
    ``gscales``), the recipe of the reading notes, section 5.3, applied row by
    row.  Returns (codes [M][K/2], scales [M][K/16], gscales float32 [M])."""
    rows = []
    for m in range(x_bits.shape[0]):
        rows.append(quantize_act_bf16(x_bits[m:m + 1], None if gscales is None else gscales[m]))
    return (np.concatenate([r[0] for r in rows]), np.concatenate([r[1] for r in rows]),
            np.array([r[2] for r in rows], dtype=np.float32))
