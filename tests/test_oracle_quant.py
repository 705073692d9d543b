"""Pins of the oracle's NVFP4 quantization recipe: special cases, exact
round trips of on-grid tensors, power-of-two scaling, a one-hot nibble-order
check, and the error bounds RNE quantization must satisfy."""

import json
import os

import numpy as np
import torch

from conftest import GOLDEN
from oracle import nvfp4_oracle as O


def _e4m3_values():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e2m1_values():
    with open(os.path.join(GOLDEN, "e2m1_codes.json")) as f:
        g = json.load(f)
    return np.array([g["codes"][str(c)] for c in range(16)])


def test_all_zero_tensor():
    x = np.zeros((3, 64), np.float32)
    x[1, 5] = -0.0
    x[2, :] = -0.0
    codes, scales, gs = O.quantize_nvfp4(x)
    assert gs == 0
    assert not scales.any()
    q = O.unpack_codes(codes)
    assert np.array_equal(q[0], np.zeros(64, np.uint8))
    assert q[1, 5] == 8 and q[1, 4] == 0
    assert np.all(q[2] == 8)


def test_one_hot_nibble_order():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    codes, _, _ = O.quantize_nvfp4(x)
    assert codes[0, 0] & 0x0F == 7 and codes[0, 0] >> 4 == 0
    x = np.zeros((1, 32), np.float32)
    x[0, 1] = -1.0
    codes, _, _ = O.quantize_nvfp4(x)
    assert codes[0, 0] & 0x0F == 0 and codes[0, 0] >> 4 == 15
    x = np.zeros((1, 32), np.float32)
    x[0, 17] = 2.0
    codes, scales, _ = O.quantize_nvfp4(x)
    assert codes[0, 8] == 0x70 and scales[0, 0] == 0 and scales[0, 1] == 0x7E


def _on_grid_tensor(rng, rows, K, s_g):
    """x = q * S * s_g with q E2M1 values, S an E4M3 value per block, and a
    +-6 in every block so that the block amax is 6 * S * s_g exactly."""
    e2m1 = _e2m1_values()
    e4m3 = _e4m3_values()
    finite = np.array([c for c in range(1, 127)])        # positive, finite scales
    nb = K // 16
    qcode = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    scode = rng.choice(finite, (rows, nb)).astype(np.uint8)
    # the global amax block: scale 448
    scode[0, 0] = 0x7E
    for r in range(rows):
        for b in range(nb):
            j = rng.integers(0, 16)
            qcode[r, b * 16 + j] = 7 if rng.random() < 0.5 else 15
    # -0 cannot come back from an exact 0 input with + sign; keep +0
    qcode[qcode == 8] = 0
    x = e2m1[qcode] * np.repeat(e4m3[scode], 16, axis=1) * s_g
    assert np.all(x.astype(np.float32) == x)                # exact in fp32
    return x.astype(np.float32), qcode, scode


def test_on_grid_round_trip_is_exact():
    rng = np.random.default_rng(11)
    for s_g in (2.0 ** -7, 2.0 ** -20, 2.0 ** 3):
        x, qcode, scode = _on_grid_tensor(rng, 4, 128, s_g)
        codes, scales, gs = O.quantize_nvfp4(x)
        assert gs == np.float32(s_g)
        assert np.array_equal(scales, scode)
        assert np.array_equal(O.unpack_codes(codes), qcode)
        assert np.array_equal(O.dequantize(codes, scales, gs), x.astype(np.float64))


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((4, 256)) * 0.3).astype(np.float32)
    x[:, 7] *= 20
    c0, s0, g0 = O.quantize_nvfp4(x)
    for k in (-30, -5, 1, 9, 40):
        ck, sk, gk = O.quantize_nvfp4((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(ck, c0) and np.array_equal(sk, s0)
        assert gk == np.float32(g0 * np.float32(2.0 ** k))


def test_global_amax_element_maps_to_six_at_scale_448():
    rng = np.random.default_rng(13)
    for _ in range(20):
        x = rng.standard_normal((3, 160)).astype(np.float32) * np.float32(rng.uniform(1e-3, 1e3))
        codes, scales, gs = O.quantize_nvfp4(x)
        r, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert scales[r, k // 16] == 0x7E
        assert O.unpack_codes(codes)[r, k] & 7 == 7
        # s_g * 2688 reproduces the amax to float32 rounding
        assert abs(float(gs) * 2688.0 - float(np.max(np.abs(x)))) <= 2 ** -22 * float(np.max(np.abs(x)))


def test_error_bounds_of_rne_quantization():
    rng = np.random.default_rng(14)
    e4m3 = _e4m3_values()
    x = rng.standard_normal((8, 512)).astype(np.float32)
    x[:, rng.choice(512, 5, replace=False)] *= 20
    codes, scales, gs = O.quantize_nvfp4(x)
    xh = O.dequantize(codes, scales, gs)
    amax_b = np.max(np.abs(x.reshape(8, 32, 16)), axis=2).astype(np.float64)
    t = amax_b / (6 * float(gs))
    S = e4m3[scales]
    normal = t >= 2.0 ** -6
    # E4M3 RNE: relative error <= 2^-4 in the normal range, <= 2^-10 absolute below
    assert np.all(np.abs(S - t)[normal] <= 2.0 ** -4 * t[normal] * (1 + 1e-6))
    assert np.all(np.abs(S - t)[~normal] <= 2.0 ** -10 * (1 + 1e-6))
    # E2M1 RNE: |x - xhat| <= half the local grid gap (in units of the element scale)
    e = np.repeat(S * float(gs), 16, axis=1)
    v = np.abs(x.astype(np.float64)) / np.where(e > 0, e, 1)
    half_gap = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    err = np.abs(x - xh)
    over6 = v > 6
    assert np.all((err <= half_gap * e * (1 + 1e-6))[~over6])
    assert np.all((np.abs(xh) == 6 * e)[over6])


def test_static_scale_rows_are_independent():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    gs = np.float32(0.0123)
    cs, ss, g = O.quantize_nvfp4(x, gs)
    assert g == gs
    for m in range(8):
        c1, s1, _ = O.quantize_nvfp4(x[m:m + 1], gs)
        assert np.array_equal(c1[0], cs[m]) and np.array_equal(s1[0], ss[m])


def test_quantized_values_are_monotone_in_x():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((1, 16 * 64)).astype(np.float32)
    codes, scales, gs = O.quantize_nvfp4(x)
    xh = O.dequantize(codes, scales, gs).reshape(64, 16)
    xb = x.reshape(64, 16)
    for b in range(64):
        o = np.argsort(xb[b], kind="stable")
        assert np.all(np.diff(xh[b][o]) >= 0)


def _bf16_rows(seed, M, K):
    x = np.random.default_rng(seed).standard_normal((M, K)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation keeps the values exactly bf16


def test_per_token_scales_equal_the_tensor_scale_when_row_maxima_agree():
    """Rows whose amax is the same value: per-token quantization gives the
    per-tensor codes, scales and (in every row) the tensor's global scale."""
    xb = _bf16_rows(31, 4, 96)
    xb[:, 7] = 0x4120                      # 10.0 in every row, above any N(0,1) draw here
    codes, scales, gs = O.quantize_act_bf16(xb)
    tc, ts, tg = O.quantize_act_bf16_per_token(xb)
    assert tg.shape == (4,) and np.all(tg.view(np.uint32) == np.float32(gs).view(np.uint32))
    assert np.array_equal(tc, codes) and np.array_equal(ts, scales)
    assert gs == np.float32(10.0) / np.float32(2688.0)


def test_per_token_scale_follows_only_its_own_row():
    """Scaling row 1 by 2^3 (exact in bf16) multiplies only its global scale
    by 8 and leaves every code and block scale as it was; an all-zero row has
    global scale 0 and zero codes without touching the other rows."""
    xb = _bf16_rows(32, 3, 160)
    c0, s0, g0 = O.quantize_act_bf16_per_token(xb)
    x2 = xb.copy()
    x2[1] = x2[1] + np.where((x2[1] & 0x7FFF) != 0, 3 << 7, 0).astype(np.uint16)  # exponent + 3
    c1, s1, g1 = O.quantize_act_bf16_per_token(x2)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    assert g1[1] == np.float32(8.0) * g0[1] and g1[0] == g0[0] and g1[2] == g0[2]
    x3 = xb.copy()
    x3[2] = 0
    c2, s2, g2 = O.quantize_act_bf16_per_token(x3)
    assert g2[2] == 0 and not c2[2].any() and not s2[2].any()
    assert np.array_equal(c2[:2], c0[:2]) and np.array_equal(g2[:2], g0[:2])
