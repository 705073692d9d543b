"""Pins of the Q+R oracle (oracle/rotation_oracle.py): the Hadamard matrices
against their textbook definition, the float32 butterfly against exact
matrix products, and hand-worked quantizations of rotated blocks."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from oracle import rotation_oracle as RO


def test_small_hadamard_matrices_are_the_textbook_ones():
    assert np.array_equal(RO.sylvester_hadamard(1), [[1]])
    assert np.array_equal(RO.sylvester_hadamard(2), [[1, 1], [1, -1]])
    assert np.array_equal(RO.sylvester_hadamard(4), [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


@pytest.mark.parametrize("R", RO.ROTATION_SIZES)
def test_hadamard_is_orthogonal_and_symmetric(R):
    h = RO.sylvester_hadamard(R)
    assert set(np.unique(h)) == {-1, 1}
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h.T, R * np.eye(R, dtype=np.int64))
    # Sylvester order: row i, column j is (-1)^popcount(i & j)
    i, j = np.indices((R, R))
    pc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(h, np.where(pc % 2 == 0, 1, -1))


@pytest.mark.parametrize("R", RO.ROTATION_SIZES)
def test_rotation_scale_is_the_nearest_float32(R):
    c = RO.rotation_scale(R)
    assert c.dtype == np.float32
    cf = Fraction(float(c))
    ulp = Fraction(float(np.spacing(c)))
    # (c - ulp/2)^2 < 1/R < (c + ulp/2)^2, exactly
    assert (cf - ulp / 2) ** 2 < Fraction(1, R) < (cf + ulp / 2) ** 2
    if R in (16, 64):
        assert cf ** 2 == Fraction(1, R)


@pytest.mark.parametrize("R", RO.ROTATION_SIZES)
def test_one_hot_rows_give_hadamard_columns(R):
    h = RO.sylvester_hadamard(R)
    c = RO.rotation_scale(R)
    for j in (0, 1, R // 2 - 1, R - 1):
        x = np.zeros((1, 2 * R), np.float32)
        x[0, R + j] = 3.0
        y = RO.rotate_blocks_f32(x, R)
        assert np.array_equal(y[0, :R], np.zeros(R, np.float32))
        expect = (np.float32(3.0) * h[:, j].astype(np.float32)) * c
        assert np.array_equal(y[0, R:], expect.astype(np.float32))


@pytest.mark.parametrize("R", RO.ROTATION_SIZES)
def test_integer_inputs_match_the_matrix_product_exactly(R):
    # small integers: every butterfly sum is exact, so the only rounding is
    # the final multiply by c, applied to the exact H x
    rng = np.random.default_rng(R)
    x = rng.integers(-8, 9, (5, 4 * R)).astype(np.float32)
    h = RO.sylvester_hadamard(R).astype(np.float64)
    exact = (x.astype(np.float64).reshape(5, 4, R) @ h.T).reshape(5, 4 * R)
    expect = (exact.astype(np.float32) * RO.rotation_scale(R)).astype(np.float32)
    assert np.array_equal(RO.rotate_blocks_f32(x, R), expect)


@pytest.mark.parametrize("R", RO.ROTATION_SIZES)
def test_float_inputs_within_the_butterfly_error_bound(R):
    rng = np.random.default_rng(7 + R)
    x = (rng.standard_normal((4, 8 * R)) * np.exp(rng.standard_normal((4, 8 * R)))).astype(np.float32)
    y = RO.rotate_blocks_f32(x, R).astype(np.float64)
    h = RO.sylvester_hadamard(R).astype(np.float64)
    ref = (x.astype(np.float64).reshape(4, 8, R) @ h.T / np.sqrt(R)).reshape(4, 8 * R)
    # log2(R) rounded stages on partial sums bounded by sum |x| of the block,
    # then one rounded multiply
    u = 2.0 ** -24
    blk = np.repeat(np.abs(x.astype(np.float64)).reshape(4, 8, R).sum(axis=2), R, axis=1).reshape(4, 8 * R)
    bound = (np.log2(R) * u * blk + u * blk) / np.sqrt(R) + u * np.abs(ref)
    assert np.all(np.abs(y - ref) <= bound)
    # a rotation keeps each block's length
    assert np.allclose(np.linalg.norm(y.reshape(-1, R), axis=1), np.linalg.norm(x.reshape(-1, R), axis=1), rtol=1e-5)


@pytest.mark.parametrize("R", [16, 64])
def test_rotation_is_an_involution(R):
    # H / sqrt(R) is symmetric and orthogonal; with c a power of two and
    # integer inputs both passes are exact
    x = np.random.default_rng(3).integers(-20, 21, (2, 3 * R)).astype(np.float32)
    assert np.array_equal(RO.rotate_blocks_f32(RO.rotate_blocks_f32(x, R), R), x)


def test_dot_products_survive_the_rotation():
    rng = np.random.default_rng(11)
    a = rng.standard_normal((3, 512)).astype(np.float32)
    w = rng.standard_normal((5, 512)).astype(np.float32)
    for R in RO.ROTATION_SIZES:
        ra, rw = RO.rotate_blocks_f32(a, R).astype(np.float64), RO.rotate_blocks_f32(w, R).astype(np.float64)
        assert np.allclose(ra @ rw.T, a.astype(np.float64) @ w.astype(np.float64).T, rtol=1e-5, atol=1e-4)


def _bf16_bits(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_hand_worked_rotated_blocks():
    # one block of 16: x = e_0 rotates to sixteen 0.25s; amax 0.25 sets
    # s_g = 0.25 / 2688, t_b = 0.25 / (6 s_g) = 448 -> code 0x7E, element
    # scale 448 s_g = 1/24, and every element 0.25 * 24 = 6 -> E2M1 code 7
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 1.0
    codes, scales, gs = RO.quantize_act_bf16_rotated(_bf16_bits(x), 16)
    assert gs == np.float32(np.float32(0.25) / np.float32(2688.0))
    assert scales.tolist() == [[0x7E]]
    assert O.unpack_codes(codes).tolist() == [[7] * 16]
    # x = e_0 + e_1: columns 0 and 1 of H_16 add to 2 where they agree (even
    # rows) and cancel elsewhere -> [0.5, 0, 0.5, 0, ...]; 0.5 maps to 6 again
    x[0, 1] = 1.0
    codes, scales, gs = RO.quantize_act_bf16_rotated(_bf16_bits(x), 16)
    assert scales.tolist() == [[0x7E]]
    assert O.unpack_codes(codes).tolist() == [[7, 0] * 8]
    # x = e_0 - e_1: odd rows survive with the sign pattern of column 1 negated
    x[0, 1] = -1.0
    codes, _, _ = RO.quantize_act_bf16_rotated(_bf16_bits(x), 16)
    assert O.unpack_codes(codes).tolist() == [[0, 7] * 8]


def test_q_plus_r_is_quantization_of_the_rotated_tensor():
    rng = np.random.default_rng(5)
    xb = _bf16_bits(rng.standard_normal((3, 256)).astype(np.float32))
    for R in RO.ROTATION_SIZES:
        got = RO.quantize_act_bf16_rotated(xb, R)
        ref = O.quantize_nvfp4(RO.rotate_blocks_f32(O.bf16_to_f32(xb), R))
        assert all(np.array_equal(g, r) for g, r in zip(got, ref))
        # a static global scale is used as given
        st = RO.quantize_act_bf16_rotated(xb, R, gscale=np.float32(0.003))
        assert st[2] == np.float32(0.003)
