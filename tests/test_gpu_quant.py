"""GPU parity of activation quantization and weight packing: codes, block
scales and global scale must be bit-identical to the oracle."""

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
import workloads as W
from oracle import nvfp4_oracle as O
from gpu_util import assert_same_q, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


def _act_case(bits, what, gscale=None):
    print(f"[quant] {what} shape={bits.shape}", flush=True)
    gs_t = None if gscale is None else torch.tensor([gscale], dtype=torch.float32, device="cuda:0")
    got = host(F.nvfp4_quantize_act(bf16_dev(bits), gscale=gs_t))
    ref = O.quantize_act_bf16(bits, gscale)
    assert_same_q(got, ref, what=what)
    return got


@pytest.mark.parametrize("K", [4096, 5120, 8192, 12288, 25600])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16, 32, 64, 128])
def test_activation_workloads(M, K):
    _act_case(W.activations_bf16(101 + K, K, M), f"act M={M} K={K}")


def test_swiglu_activation():
    for M in (1, 8):
        _act_case(W.swiglu_activations_bf16(1213, 1223, 12288, M), f"swiglu M={M}")


def _tie_tensor(M, K, seed):
    """bf16 tensor whose elements land exactly on E2M1 midpoints and whose
    block amaxes land exactly on E4M3 midpoints (power-of-two global scale)."""
    rng = np.random.default_rng(seed)
    s_g = 2.0 ** -7                       # amax 21 -> s_g = 21/2688 = 2^-7 exactly
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 3.0, 0.0])
    e4m3_mid_blocks = np.array([1.0625, 1.1875, 3.25, 0.0029296875, 17.0, 448.0, 0.001953125, 0.0009765625])
    x = np.zeros((M, K))
    for m in range(M):
        for b in range(K // 16):
            S = rng.choice(e4m3_mid_blocks)
            blk = rng.choice(mids, 16) * rng.choice([-1.0, 1.0], 16)
            blk[rng.integers(0, 16)] = 6.0 * (1 if rng.random() < 0.5 else -1)
            x[m, b * 16:(b + 1) * 16] = blk * S * s_g
    x[0, 0] = 21.0                        # the global amax: 6 * 448 * 2^-7
    f = x.astype(np.float32)
    bits = W.to_bf16_bits(f)
    assert np.array_equal(W.bf16_bits_to_f32(bits), f), "tie tensor must be exact in bf16"
    return bits


def test_rne_ties_on_both_grids():
    for M, K in [(1, 512), (8, 1024), (8, 8192)]:
        _act_case(_tie_tensor(M, K, 5 + K), f"ties M={M} K={K}")


def test_special_tensors():
    K = 256
    z = np.zeros((2, K), np.uint16)
    _act_case(z, "all +0")
    z[1, ::3] = 0x8000                     # -0.0
    _act_case(z, "signed zeros")
    one = np.zeros((1, K), np.uint16); one[0, 77] = W.to_bf16_bits(np.array([-3.5], np.float32))[0]
    _act_case(one, "single nonzero")
    rng = np.random.default_rng(9)
    tiny = rng.integers(1, 0x0080, (4, K)).astype(np.uint16)     # bf16 subnormals
    tiny |= (rng.integers(0, 2, (4, K)) << 15).astype(np.uint16)
    _act_case(tiny, "bf16 subnormals")
    huge = W.to_bf16_bits((rng.standard_normal((3, K)) * 1e37).astype(np.float32))
    _act_case(huge, "huge magnitudes")
    wide = W.to_bf16_bits((rng.standard_normal((2, K)) * np.exp2(rng.uniform(-60, 60, (2, K)))).astype(np.float32))
    _act_case(wide, "wide dynamic range")


def test_static_scale_and_row_independence():
    bits = W.activations_bf16(77, 5120, 8)
    gs = np.float32(0.0371)
    full = _act_case(bits, "static M=8", gscale=gs)
    for m in (0, 5):
        one = _act_case(bits[m:m + 1], f"static row {m}", gscale=gs)
        assert np.array_equal(one[0][0], full[0][m]) and np.array_equal(one[1][0], full[1][m])


def test_quantize_is_repeatable():
    x = bf16_dev(W.activations_bf16(55, 25600, 8))
    a = host(F.nvfp4_quantize_act(x))
    b = host(F.nvfp4_quantize_act(x))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


@pytest.mark.parametrize("N,K", [(1000, 512), (333, 96), (4096, 4096), (6144, 4096)])
def test_pack_small_and_8b_shapes_full_compare(N, K):
    print(f"[pack] N={N} K={K}", flush=True)
    w = W.weights(1234 + N, N, K, outlier_rows=True)
    got = host(F.nvfp4_pack_weights(f32_dev(w)))
    assert_same_q(got, O.quantize_nvfp4(w), what=f"pack {N}x{K}")


@pytest.mark.parametrize("case", W.qwen3_32b_cases() + [W.lm_head_case()], ids=lambda c: c.name)
def test_pack_full_size_sampled_rows(case):
    print(f"[pack] {case.name} {case.N}x{case.K}", flush=True)
    w = W.weights(case.w_seed, case.N, case.K, case.w_outlier_rows)
    wt = f32_dev(w)
    got = host(F.nvfp4_pack_weights(wt))
    del wt
    torch.cuda.empty_cache()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, case.N - 1], W.outlier_rows_of(case.w_seed, case.N, case.K)[:8],
                                     rng.choice(case.N, 48, replace=False)]))
    s_g = O.global_scale(np.max(np.abs(w)))
    ref = O.quantize_nvfp4(w[rows], s_g)
    assert_same_q(got, ref, rows=rows, what=case.name)
