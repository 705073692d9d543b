"""GPU parity of per-token activation global scales: the quantization is
bit-identical to the oracle's row-by-row recipe (dynamic and static), and
the GEMV with one scale per token, through every compiled kernel variant and
the LM-head epilogue, is within |y - y_ref| <= 1e-5 * sum_k |a_k w_k| of the
oracle's exact result."""

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
import workloads as W
from oracle import nvfp4_oracle as O
from oracle import reset_oracle as R
from gpu_util import assert_gemv_close, bf16_dev, f32_dev

pytestmark = pytest.mark.gpu


def _host_pt(q: F.NvFp4Tensor):
    torch.cuda.synchronize()
    return q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.gscale.cpu().numpy().astype(np.float32)


def _same(got, ref, what):
    gc, gs, gg = got
    rc, rs, rg = ref
    assert np.array_equal(gg.view(np.uint32), np.asarray(rg, np.float32).view(np.uint32)), (what, gg, rg)
    assert np.array_equal(gc, rc), (what, "codes differ at", np.argwhere(gc != rc)[:5])
    assert np.array_equal(gs, rs), (what, "scales differ at", np.argwhere(gs != rs)[:5])


def _spread_rows(bits, seed):
    """Scale row m by 2^e_m (exact in bf16) so that the rows' maxima differ."""
    e = np.random.default_rng(seed).integers(-6, 7, bits.shape[0])
    out = bits.copy()
    for m, k in enumerate(e):
        nz = (out[m] & 0x7FFF) != 0
        out[m] = np.where(nz, (out[m].astype(np.int32) + (int(k) << 7)).astype(np.uint16), out[m])
    return out


@pytest.mark.parametrize("M,K", [(1, 32), (2, 160), (3, 4128), (8, 5120), (8, 25600), (16, 8192), (64, 12288),
                                 (128, 5120), (5, 131072)])
def test_dynamic_token_scales_bit_exact(M, K):
    print(f"[token quant] M={M} K={K}", flush=True)
    xb = _spread_rows(W.activations_bf16(300 + K, K, M), 7 + M)
    xb[M // 2] = 0  # an all-zero row: scale 0, codes 0
    got = _host_pt(F.nvfp4_quantize_act(bf16_dev(xb), per_token=True))
    _same(got, O.quantize_act_bf16_per_token(xb), f"M={M} K={K}")


def test_static_token_scales_bit_exact():
    M, K = 8, 5120
    xb = _spread_rows(W.activations_bf16(310, K, M), 11)
    gs = np.array([0.01, 0.02, 0.5, 1e-3, 0.07, 0.3, 2.0, 0.004], np.float32)
    got = _host_pt(F.nvfp4_quantize_act(bf16_dev(xb), gscale=torch.from_numpy(gs).to("cuda:0"), per_token=True))
    _same(got, O.quantize_act_bf16_per_token(xb, gs), "static")


# one shape every variant runs (K % 256 == 0, small enough for every LDS layout)
@pytest.mark.parametrize("variant", F.nvfp4_gemv_variant_names() if __import__("os").path.exists(F.LIB_PATH) else [])
def test_every_kernel_variant_with_token_scales(variant):
    mt = F.variant_tokens(variant)
    with F.forced_variant(variant):
        _token_variant_case(variant, mt)


def _token_variant_case(variant, mt):
    N, K = 300, 5120
    w = W.small_random_weights(N + 5, N, K)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    wr = O.quantize_nvfp4(w)
    for M in sorted({max(1, mt - 1), mt}):
        assert F.nvfp4_gemv_variant(M, N, K) == variant
        print(f"[token gemv] {variant} M={M} N={N} K={K}", flush=True)
        xb = _spread_rows(W.small_random_bf16(3 * M + 1, M, K), M)
        aq = F.nvfp4_quantize_act(bf16_dev(xb), per_token=True)
        y = F.nvfp4_gemv_smallm(aq, wq)
        torch.cuda.synchronize()
        ar = O.quantize_act_bf16_per_token(xb)
        y_ref, ref_abs = O.gemv_ref(ar, wr)
        assert_gemv_close(y.cpu().numpy(), y_ref, ref_abs, what=f"{variant} M={M}")


@pytest.mark.parametrize("M", [1, 2, 4, 8, 32])
def test_full_size_projection_with_token_scales(M):
    case = [c for c in W.qwen3_32b_cases() if c.name.endswith("gate_up")][0]
    print(f"[token gemv] {case.name} M={M}", flush=True)
    w = W.weights(case.w_seed, case.N, case.K, case.w_outlier_rows)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    rows = np.unique(np.concatenate([[0, case.N - 1], np.random.default_rng(4).choice(case.N, 40, replace=False)]))
    wr = O.quantize_nvfp4(w[rows], O.global_scale(np.max(np.abs(w))))
    del w
    xb = _spread_rows(W.case_activations_bf16(case, M), 20 + M)
    y = F.nvfp4_gemv_smallm(F.nvfp4_quantize_act(bf16_dev(xb), per_token=True), wq)
    torch.cuda.synchronize()
    y_ref, ref_abs = O.gemv_ref(O.quantize_act_bf16_per_token(xb), wr)
    assert_gemv_close(y.cpu().numpy()[:, rows], y_ref, ref_abs, what=f"gate_up M={M}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_lm_head_epilogue_with_token_scales(M):
    """Entropies from logits computed with per-token scales: within 1e-4
    nats of the fp64 entropy of the GPU's own logits; logits against the
    oracle."""
    dev = torch.device("cuda:0")
    N, K = 20000, 1024
    w = W.small_random_weights(61, N, K, scale=0.2)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    xb = _spread_rows(W.small_random_bf16(62, M, K), 63)
    aq = F.nvfp4_quantize_act(bf16_dev(xb), per_token=True)
    st = F.new_reset_state(M, 4, dev)
    ent, tmp = torch.empty(M, device=dev), torch.empty(M, device=dev)
    flags = torch.ones(M, dtype=torch.uint8, device=dev)
    ws = F.new_workspace(F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, M, N, K), dev)
    y = F.nvfp4_gemv_smallm(aq, wq, epi=F.Epilogue(flags, st, ent, tmp, window=4), ws=ws)
    torch.cuda.synchronize()
    logits = y.cpu().numpy()
    Href = R.entropy_rows(logits.astype(np.float64))
    assert np.all(np.abs(ent.cpu().numpy() - Href) <= 1e-4), (ent.cpu().numpy(), Href)
    y_ref, ref_abs = O.gemv_ref(O.quantize_act_bf16_per_token(xb), O.quantize_nvfp4(w))
    assert_gemv_close(logits, y_ref, ref_abs, what=f"lm M={M}")


def test_graph_replays_match_eager():
    """Per-token quantization + GEMV captured in a HIP graph and replayed
    with a new activation before each replay (eager work in between) gives
    the eager bits every time."""
    M, N, K = 8, 6000, 5120
    w = W.small_random_weights(71, N, K)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    xs = [bf16_dev(_spread_rows(W.small_random_bf16(72 + i, M, K), 73 + i)) for i in range(3)]
    ref = []
    for xi in xs:
        aq = F.nvfp4_quantize_act(xi, per_token=True)
        ref.append((F.nvfp4_gemv_smallm(aq, wq).clone(), aq.gscale.clone()))
    x = torch.empty_like(xs[0])
    aq = F.nvfp4_quantize_act(xs[0], per_token=True)
    y = torch.empty((M, N), device=x.device)
    s = torch.cuda.Stream()

    def call():
        F.nvfp4_quantize_act(x, out=aq, stream=s, per_token=True)
        F.nvfp4_gemv_smallm(aq, wq, y=y, stream=s)

    with torch.cuda.stream(s):
        x.copy_(xs[0])
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for r in range(6):
        x.copy_(xs[r % 3])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[r % 3][0]), r
        assert torch.equal(aq.gscale, ref[r % 3][1]), r
        y.zero_()
        torch.cuda.synchronize()
