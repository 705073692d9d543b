"""The seeded input generators are deterministic and consistent with the
stated recipe (shapes, outlier counts, row-streamed generation)."""

import numpy as np

import workloads as W


def test_weight_rows_match_full_draw():
    full = W.weights(5, 300, 64, outlier_rows=True)
    rows = np.array([299, 0, 17, 150, 17])
    part = W.weight_rows(5, 300, 64, True, rows)
    assert np.array_equal(part, full[rows])
    orows = W.outlier_rows_of(5, 300, 64)
    assert len(orows) == 0   # floor(0.001*300) == 0
    full2 = W.weights(6, 3000, 32, outlier_rows=True)
    orows = W.outlier_rows_of(6, 3000, 32)
    assert len(orows) == 3
    base = W.weights(6, 3000, 32, outlier_rows=False)
    assert np.array_equal(full2[orows], base[orows] * np.float32(8))


def test_activation_recipe():
    x = W.activations_f32(9, 4096)
    big = np.abs(x).max(axis=0) > 10
    assert x.shape == (8, 4096)
    b = W.activations_bf16(9, 4096, 2)
    assert b.shape == (2, 4096) and b.dtype == np.uint16
    assert np.array_equal(W.activations_bf16(9, 4096, 8)[:2], b)
    f = W.bf16_bits_to_f32(b)
    assert np.all(np.abs(f - x[:2]) <= np.abs(x[:2]) * 2 ** -8)
    assert 30 <= big.sum() <= 40


def test_step_flags_and_cases():
    f = W.step_flags(3300, 512, 8)
    assert f.shape == (512, 8) and np.all(f[0] == 1)
    assert 0.005 < f[1:].mean() < 0.05
    cases = W.qwen3_32b_cases()
    assert [(c.N, c.K) for c in cases] == [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)]
    assert W.qwen3_8b_cases()[3].swiglu


def test_sampler_uniforms():
    u = W.sampler_uniforms(3500, 4, 8)
    assert u.shape == (4, 8) and u.dtype == np.float32
    assert np.all((u >= 0) & (u < 1))
    assert np.array_equal(W.sampler_uniforms(3500, 4, 3), u[:, :3])   # fewer sequences: a prefix
    assert not np.array_equal(W.sampler_uniforms(3501, 4, 8), u)
