"""GPU parity of the small-M GEMV against the oracle: every output within
|y - y_ref| <= 1e-5 * sum_k |a_k w_k| (the oracle's exact fp64 result)."""

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
import workloads as W
from oracle import nvfp4_oracle as O
from gpu_util import assert_gemv_close, assert_same_q, bf16_dev, f32_dev, host, oracle_rows_ref

pytestmark = pytest.mark.gpu


def _run(M, N, K, w, xbits, what):
    print(f"[gemv] {what} M={M} N={N} K={K}", flush=True)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    aq = F.nvfp4_quantize_act(bf16_dev(xbits))
    y = F.nvfp4_gemv_smallm(aq, wq)
    torch.cuda.synchronize()
    return wq, aq, y.cpu().numpy()


# small shapes: several tiles, ragged row tails, K that is not a multiple of
# the lane stride, multi-phase K for larger M
SMALL = [(1, 1, 32), (1, 100, 64), (2, 257, 96), (3, 33, 160), (4, 1000, 512), (5, 64, 4096),
         (6, 129, 4128), (7, 70, 8192), (8, 500, 5120), (8, 17, 12288), (8, 300, 25600), (1, 4097, 4096),
         (9, 300, 5120), (11, 1000, 512), (12, 129, 4128), (16, 37, 96), (16, 515, 8192), (16, 70, 25600),
         (17, 300, 5120), (24, 129, 4128), (31, 1000, 512), (32, 37, 96), (32, 515, 8192), (32, 70, 25600),
         (33, 300, 5120), (48, 129, 4128), (64, 37, 96), (64, 515, 8192), (64, 70, 25600),
         (65, 300, 5120), (100, 129, 4128), (128, 37, 96), (128, 515, 2048), (128, 70, 25600)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_shapes_full_compare(M, N, K):
    w = W.small_random_weights(N * 7 + K, N, K)
    xb = W.small_random_bf16(M * 13 + K, M, K)
    wq, aq, y = _run(M, N, K, w, xb, "small")
    wr, ar = O.quantize_nvfp4(w), O.quantize_act_bf16(xb)
    assert_same_q(host(wq), wr, what="pack")
    assert_same_q(host(aq), ar, what="act")
    y_ref, ref_abs = O.gemv_ref(ar, wr)
    assert_gemv_close(y, y_ref, ref_abs, what=f"M={M} N={N} K={K}")


# the tiled GEMM as the launch table picks it (17..128 tokens, N >= 16384):
# a ragged last 128-row tile, one stage and many stages of K, tokens below
# and at each compiled token count
GEMM_DEFAULT = [(17, 16500, 256), (32, 16500, 4352), (33, 16389, 1024), (64, 16389, 4352), (100, 16500, 512),
                (128, 16389, 2304)]


@pytest.mark.parametrize("M,N,K", GEMM_DEFAULT)
def test_gemm_default_full_compare(M, N, K):
    assert F.nvfp4_gemv_variant(M, N, K).startswith("gemm_m")
    w = W.small_random_weights(N * 3 + K + M, N, K)
    xb = W.small_random_bf16(M * 17 + K, M, K)
    wq, aq, y = _run(M, N, K, w, xb, F.nvfp4_gemv_variant(M, N, K))
    y_ref, ref_abs = O.gemv_ref(O.quantize_act_bf16(xb), O.quantize_nvfp4(w))
    assert_gemv_close(y, y_ref, ref_abs, what=f"gemm M={M} N={N} K={K}")


# the tiled GEMM split along K (65..128 tokens, K >= 16384, few row tiles):
# partial sums in the workspace, then the in-order reduce; ragged last tile
SPLIT_DEFAULT = [(65, 1000, 16384), (128, 777, 16640), (100, 5120, 16384)]


@pytest.mark.parametrize("M,N,K", SPLIT_DEFAULT)
def test_gemm_split_default_full_compare(M, N, K):
    assert F.nvfp4_gemv_variant(M, N, K) == "gemm_m128"
    assert F.nvfp4_workspace_size(F.NVFP4_OP_GEMV, M, N, K) > 0
    w = W.small_random_weights(N * 7 + K + M, N, K)
    xb = W.small_random_bf16(M * 23 + K, M, K)
    wq, aq, y = _run(M, N, K, w, xb, F.nvfp4_gemv_variant(M, N, K))
    y_ref, ref_abs = O.gemv_ref(O.quantize_act_bf16(xb), O.quantize_nvfp4(w))
    assert_gemv_close(y, y_ref, ref_abs, what=f"split gemm M={M} N={N} K={K}")


# the wave-owned streaming kernel as the launch table picks it (LM-head-sized
# N >= 65536 without the epilogue): 2 tokens with the activation read from
# L2, 3..4 tokens with it staged in LDS, with a ragged last 48-row workgroup
# and a ragged last 12-row wave block
WSTREAM_DEFAULT = [(2, 65600, 1024, "wstream_m4_r3_w4_u2_ag"), (3, 65601, 512, "wstream_m4_r3_w4_u2"),
                   (4, 65557, 1024, "wstream_m4_r3_w4_u2")]


@pytest.mark.parametrize("M,N,K,variant", WSTREAM_DEFAULT)
def test_wstream_default_full_compare(M, N, K, variant):
    assert F.nvfp4_gemv_variant(M, N, K) == variant
    w = W.small_random_weights(N * 5 + K + M, N, K)
    xb = W.small_random_bf16(M * 19 + K, M, K)
    wq, aq, y = _run(M, N, K, w, xb, F.nvfp4_gemv_variant(M, N, K))
    y_ref, ref_abs = O.gemv_ref(O.quantize_act_bf16(xb), O.quantize_nvfp4(w))
    assert_gemv_close(y, y_ref, ref_abs, what=f"wstream M={M} N={N} K={K}")


def _full_size(case, Ms):
    w = W.weights(case.w_seed, case.N, case.K, case.w_outlier_rows)
    wt = f32_dev(w)
    wq = F.nvfp4_pack_weights(wt)
    del wt
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, 1, case.N - 1], W.outlier_rows_of(case.w_seed, case.N, case.K)[:6],
                                     rng.choice(case.N, 60, replace=False)]))
    s_g = O.global_scale(np.max(np.abs(w)))
    wr = O.quantize_nvfp4(w[rows], s_g)
    del w
    for M in Ms:
        xb = W.case_activations_bf16(case, M)
        print(f"[gemv] {case.name} M={M} N={case.N} K={case.K}", flush=True)
        aq = F.nvfp4_quantize_act(bf16_dev(xb))
        y = F.nvfp4_gemv_smallm(aq, wq)
        torch.cuda.synchronize()
        ar = O.quantize_act_bf16(xb)
        assert_same_q(host(aq), ar, what=f"act {case.name} M={M}")
        y_ref, ref_abs = O.gemv_ref(ar, wr)
        assert_gemv_close(y.cpu().numpy()[:, rows], y_ref, ref_abs, what=f"{case.name} M={M}")


def test_single_4096_full_compare():
    case = W.single_case()
    w = W.weights(case.w_seed, case.N, case.K)
    xb = W.activations_bf16(case.x_seed, case.K, 1)
    wq, aq, y = _run(1, case.N, case.K, w, xb, case.name)
    wr, ar = O.quantize_nvfp4(w), O.quantize_act_bf16(xb)
    y_ref, ref_abs = O.gemv_ref(ar, wr)
    assert_gemv_close(y, y_ref, ref_abs, what=case.name)


@pytest.mark.parametrize("case", W.qwen3_8b_cases(), ids=lambda c: c.name)
def test_qwen3_8b_projections(case):
    _full_size(case, (1, 2, 4, 8))


@pytest.mark.parametrize("case", W.qwen3_32b_cases(), ids=lambda c: c.name)
def test_qwen3_32b_projections(case):
    _full_size(case, (1, 2, 4, 8, 16, 32, 64, 128))


def test_lm_head_projection():
    _full_size(W.lm_head_case(), (1, 8))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", W.qwen3_32b_cases(), ids=lambda c: c.name)
def test_qwen3_32b_every_row(case):
    """Every output row of the full-size Qwen3-32B projections at M = 1 and
    8, against the oracle's own quantization and fp64 GEMV of the whole
    weight matrix (row chunks)."""
    w = W.weights(case.w_seed, case.N, case.K, case.w_outlier_rows)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    s_g = O.global_scale(np.max(np.abs(w)))
    xb = W.case_activations_bf16(case, 8)
    ys = {}
    for M in (1, 8):
        print(f"[gemv rows] {case.name} M={M} N={case.N} K={case.K}", flush=True)
        aq = F.nvfp4_quantize_act(bf16_dev(xb[:M]))
        ys[M] = F.nvfp4_gemv_smallm(aq, wq).cpu().numpy()
    refs = oracle_rows_ref(w, s_g, [O.quantize_act_bf16(xb[:1]), O.quantize_act_bf16(xb)])
    for (M, (y_ref, ref_abs)) in zip((1, 8), refs):
        assert_gemv_close(ys[M], y_ref, ref_abs, what=f"{case.name} M={M} all rows")


def test_zero_activation_and_zero_rows():
    N, K = 300, 1024
    w = W.small_random_weights(3, N, K)
    w[7] = 0.0
    w[299] = -0.0
    xb = W.small_random_bf16(4, 4, K)
    xb[2] = 0
    wq, aq, y = _run(4, N, K, w, xb, "zeros")
    assert np.all(y[2] == 0.0)
    assert np.all(y[:, 7] == 0.0) and np.all(y[:, 299] == 0.0)


def test_gemv_is_repeatable_and_rows_do_not_depend_on_m():
    N, K = 5120, 8192
    w = W.small_random_weights(11, N, K)
    xb = W.small_random_bf16(12, 8, K)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    gs = torch.tensor([0.01], dtype=torch.float32, device="cuda:0")      # static: rows independent
    aq8 = F.nvfp4_quantize_act(bf16_dev(xb), gscale=gs)
    y1 = F.nvfp4_gemv_smallm(aq8, wq).cpu().numpy()
    y2 = F.nvfp4_gemv_smallm(aq8, wq).cpu().numpy()
    assert np.array_equal(y1, y2)
    aq1 = F.nvfp4_quantize_act(bf16_dev(xb[:1]), gscale=gs)
    y3 = F.nvfp4_gemv_smallm(aq1, wq).cpu().numpy()
    # same inputs for row 0; results agree to the tolerance (tilings differ by M)
    wr = O.quantize_nvfp4(w)
    ar = O.quantize_act_bf16(xb[:1], np.float32(0.01))
    y_ref, ref_abs = O.gemv_ref(ar, wr)
    assert_gemv_close(y3, y_ref, ref_abs, what="M=1 static")
    assert_gemv_close(y1[:1], y_ref, ref_abs, what="M=8 row 0 static")


VARIANT_SHAPES = [(1, 37, 160), (16, 515, 4128), (16, 300, 5120), (16, 129, 25600)]
# kernels that need K % 256 == 0: one step, 17 steps over the waves, two full sizes
VARIANT_SHAPES_K256 = [(1, 37, 256), (16, 515, 4352), (16, 300, 5120), (16, 129, 25600)]
# ... K % 512 == 0: one chunk, 9 chunks over the waves, two full sizes
VARIANT_SHAPES_K512 = [(1, 37, 512), (16, 515, 4608), (16, 300, 5120), (16, 129, 25600)]


@pytest.fixture
def force():
    """forced_variant(...) for the test's duration; the launch table is
    restored afterwards."""
    yield F.forced_variant
    F.nvfp4_gemv_tune(None, True)


@pytest.mark.parametrize("variant", F.nvfp4_gemv_variant_names() if __import__("os").path.exists(F.LIB_PATH) else [])
def test_every_kernel_variant(variant, force):
    """Each compiled variant (forced through nvfp4_gemv_tune) against the
    oracle: ragged row tails, K not a multiple of 128, several K phases, and
    M below and at the variant's token count.  A variant whose LDS would not
    fit a shape is not launched there (the default runs instead); every
    variant runs at least two of the shapes."""
    mt = F.variant_tokens(variant)
    force(variant).__enter__()
    shapes = {32: VARIANT_SHAPES, 256: VARIANT_SHAPES_K256, 512: VARIANT_SHAPES_K512}[F.variant_k_multiple(variant)]
    ran = 0
    for M in sorted({1, max(1, mt - 1), mt}):
        for (nmul, N, K) in shapes:
            if F.nvfp4_gemv_variant(M, N, K) != variant:
                assert K >= 25600, (variant, M, N, K)  # only the largest K may exceed a variant's LDS
                continue
            ran += 1
            w = W.small_random_weights(N + K + M, N, K)
            xb = W.small_random_bf16(3 * N + M, M, K)
            wq, aq, y = _run(M, N, K, w, xb, variant)
            y_ref, ref_abs = O.gemv_ref(O.quantize_act_bf16(xb), O.quantize_nvfp4(w))
            assert_gemv_close(y, y_ref, ref_abs, what=f"{variant} M={M} N={N} K={K}")
    assert ran >= 2, variant


# Row mapping of the MFMA tile kernels: whole tiles (forced with
# nvfp4_gemv_tune(..., balance=False)) against rows dealt out evenly over the CUs (the
# default where whole tiles would leave CUs idle; N = 5120 gives 20 or 10
# rows per workgroup).  N = 4099 leaves a ragged last tile in both mappings;
# N = 5120 - 3 a ragged last workgroup of the even deal.
ROW_MAP_CASES = [("lmfma_m8_r2_w8_p1", 8, 4099, 2048), ("lmfma_m8_r1_w4_p1", 5, 5117, 1280),
                 ("lmfma_m16_r2_w8_p1", 16, 5117, 2048), ("lmfma_m16_r1_w4_p1", 10, 4099, 1312),
                 ("lmfma_m32_r2_w8_p1", 32, 5117, 2048), ("lmfma_m32_r1_w4_p1", 20, 4099, 1312),
                 ("lmfma_m64_r2_w8_p1", 64, 5117, 2048), ("lmfma_m64_r2_w4_p1", 40, 4099, 1312),
                 ("lmfma_m128_r1_w4_p1", 128, 5117, 1024), ("lmfma_m128_r2_w4_p1", 90, 4099, 1312),
                 ("dma_m8_r2_w4_d3", 8, 5117, 1024), ("stream8_m8_r5_w4_u2", 7, 4099, 2048),
                 ("stream8_m8_r3_w8_u2", 6, 5117, 2048), ("stream8_m8_r2_w4_u2", 5, 4099, 1280),
                 ("fmma_m4_r2_w4_d3", 4, 5117, 1024), ("fmma_m2_r1_w4_d3_sa", 2, 4099, 1024),
                 ("stream8_m8_r3_w4_u2", 8, 5117, 1024), ("stream_m4_r5_w4_u2", 3, 4099, 2048),
                 ("stream8_m16_r5_w4_u2", 16, 4099, 2048), ("stream8_m16_r4_w4_u2", 11, 5117, 1024)]


@pytest.mark.parametrize("balance", ["0", "1"])
@pytest.mark.parametrize("variant,M,N,K", ROW_MAP_CASES)
def test_row_mapping(variant, M, N, K, balance, force):
    force(variant, balance == "1").__enter__()
    assert F.nvfp4_gemv_variant(M, N, K) == variant
    w = W.small_random_weights(N + 5 * K, N, K)
    xb = W.small_random_bf16(N + M, M, K)
    wq, aq, y = _run(M, N, K, w, xb, f"{variant} balance={balance}")
    y_ref, ref_abs = O.gemv_ref(O.quantize_act_bf16(xb), O.quantize_nvfp4(w))
    assert_gemv_close(y, y_ref, ref_abs, what=f"{variant} balance={balance} M={M} N={N} K={K}")
