"""CPU oracle for the rotation-fused activation quantization ("Q+R").

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it and shares no code, table or constant generator with it.

What it computes, and where that comes from:

* The reading notes (Paper-Reading-Collection, section 5.3 and its Table 3)
  compare the plain per-layer activation quantization "Q" with the
  rotation-fused quantization "Q+R" of rotation-based NVFP4 pipelines
  (MR-GPTQ, block-rotation BRQ), which costs about 2.3x Q at M = 1.  The
  pages give no rotation size or formula.
* Reading taken (listed in the design notes): the rotation is the
  normalized Walsh-Hadamard transform H_R / sqrt(R) applied to every run of
  R consecutive elements of each row (block-diagonal), R a power of two in
  {16, 32, 64, 128}; R = 16 is one NVFP4 scale block.  H_R is Sylvester's
  matrix (H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]).  The rotated
  activation is then quantized with the unchanged NVFP4 recipe of
  ``nvfp4_oracle``.  Weights rotated the same way give the same projection,
  since (A Q)(W Q)^T = A W^T for the orthogonal Q = H_R / sqrt(R).
* The rotation's rounding is fixed in float32 because its output decides
  quantized codes: butterfly stages h = 1, 2, 4, ..., R/2 in that order,
  each pair (i, i + h) with i & h == 0 becoming (fl(a + b), fl(a - b)), then
  one multiply by c = the float32 nearest to 1/sqrt(R).
"""

from __future__ import annotations

import numpy as np

from oracle import nvfp4_oracle as O

ROTATION_SIZES = (16, 32, 64, 128)


def sylvester_hadamard(n: int) -> np.ndarray:
    """The n x n Sylvester Hadamard matrix (entries +-1), n a power of two."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_scale(R: int) -> np.float32:
    """c = the float32 nearest to 1/sqrt(R) (exact for R = 16 and 64)."""
    return np.float32(1.0 / np.sqrt(np.float64(R)))


def rotate_blocks_f32(x: np.ndarray, R: int) -> np.ndarray:
    """(H_R / sqrt(R)) applied to each run of R consecutive elements of every
    row of the float32 matrix x [rows][K] (K % R == 0), by the float32
    butterfly described in the module docstring."""
    if R not in ROTATION_SIZES:
        raise ValueError(f"R must be one of {ROTATION_SIZES}")
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % R:
        raise ValueError("K must be a multiple of R")
    y = x.reshape(rows, K // R, R).copy()
    h = 1
    while h < R:
        # pairs (i, i + h) with i & h == 0: view the block as [R / 2h][2][h]
        v = y.reshape(rows, K // R, R // (2 * h), 2, h)
        a = v[:, :, :, 0, :].copy()
        b = v[:, :, :, 1, :].copy()
        v[:, :, :, 0, :] = (a + b).astype(np.float32)
        v[:, :, :, 1, :] = (a - b).astype(np.float32)
        h *= 2
    y = (y * rotation_scale(R)).astype(np.float32)
    return y.reshape(rows, K)


def quantize_act_bf16_rotated(x_bits: np.ndarray, R: int, gscale: float | None = None):
    """Q+R: rotate the bf16 activation [M][K] (bit patterns) by blocks of R,
    then quantize it with the NVFP4 recipe (dynamic global scale from the
    rotated tensor's amax, or the given static one)."""
    return O.quantize_nvfp4(rotate_blocks_f32(O.bf16_to_f32(x_bits), R), gscale)
