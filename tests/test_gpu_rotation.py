"""GPU parity of the rotation-fused activation quantization (Q+R): codes,
block scales and global scale bit-identical to the oracle's float32 block
Walsh-Hadamard rotation followed by the NVFP4 recipe, on every rotation size,
the one-launch and two-launch dynamic paths and a static scale; and a
projection on rotated operands."""

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
import workloads as W
from oracle import nvfp4_oracle as O
from oracle import rotation_oracle as RO
from gpu_util import assert_gemv_close, assert_same_q, bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu

# (M, K): one block row, decode shapes of the one-launch path up to its
# 131072-element limit, and the two-launch path above it
SHAPES = [(1, 128), (1, 5120), (3, 4224), (8, 5120), (4, 25600), (16, 8192), (8, 25600), (64, 4096)]


def _case(bits, R, what, gscale=None):
    print(f"[q+r] {what} R={R} shape={bits.shape} static={gscale is not None}", flush=True)
    gs_t = None if gscale is None else torch.tensor([gscale], dtype=torch.float32, device="cuda:0")
    got = host(F.nvfp4_quantize_act_rotated(bf16_dev(bits), R, gscale=gs_t))
    ref = RO.quantize_act_bf16_rotated(bits, R, gscale)
    assert_same_q(got, ref, what=f"{what} R={R}")


@pytest.mark.parametrize("R", RO.ROTATION_SIZES)
@pytest.mark.parametrize("M,K", SHAPES)
def test_rotated_quantization_bit_exact(M, K, R):
    if K % R:
        pytest.skip("K is not a multiple of the rotation")
    bits = W.activations_bf16(500 + K + R, K, M)
    _case(bits, R, f"act M={M} K={K}")


@pytest.mark.parametrize("R", RO.ROTATION_SIZES)
def test_rotated_quantization_static_scale(R):
    bits = W.activations_bf16(600 + R, 5120, 8)
    _case(bits, R, "static", gscale=np.float32(0.0071))


@pytest.mark.parametrize("R", RO.ROTATION_SIZES)
def test_rotated_quantization_special_rows(R):
    """A zero row, a row of signed zeros, one-hot rows (every rotated element
    equal in magnitude) and a row spanning a wide bf16 range."""
    K = 1024
    f = np.zeros((6, K), np.float32)
    f[1, :] = -0.0
    f[2, 0] = 1.0
    f[3, R - 1] = -3.5
    f[3, R] = 2.0
    rng = np.random.default_rng(R)
    f[4] = rng.standard_normal(K) * np.exp2(rng.integers(-30, 30, K))
    f[5] = rng.standard_normal(K) * 1e-30
    _case(W.to_bf16_bits(f), R, "special")


def test_projection_on_rotated_operands():
    """y = Q+R(x) . pack(rotate(W))^T on the GPU equals the oracle's exact
    product of the same quantized operands (to the GEMV tolerance), and
    approximates the unrotated x W^T."""
    M, N, K, R = 8, 777, 4096, 16
    xb = W.activations_bf16(700, K, M)
    w = W.small_random_weights(701, N, K)
    wr = RO.rotate_blocks_f32(w, R)
    wq = F.nvfp4_pack_weights(f32_dev(wr))
    aq = F.nvfp4_quantize_act_rotated(bf16_dev(xb), R)
    y = F.nvfp4_gemv_smallm(aq, wq)
    torch.cuda.synchronize()
    a_ref = RO.quantize_act_bf16_rotated(xb, R)
    w_ref = O.quantize_nvfp4(wr)
    assert_same_q(host(aq), a_ref, what="rotated act")
    assert_same_q(host(wq), w_ref, what="rotated weights")
    y_ref, ref_abs = O.gemv_ref(a_ref, w_ref)
    yg = y.cpu().numpy()
    assert_gemv_close(yg, y_ref, ref_abs, what="rotated projection")
    exact = O.bf16_to_f32(xb).astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(yg - exact) / np.linalg.norm(exact)
    assert rel < 0.2, rel
