"""The C-ABI library loads, exports every function include/nvfp4.h declares,
and rejects bad arguments with the documented status before any HIP call
(so these run without a GPU; fake device addresses are never dereferenced)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

F = pytest.importorskip("fp4_decode_gemv_amd")

HDR = os.path.join(ROOT, "include", "nvfp4.h")
PROBE_HDR = os.path.join(ROOT, "include", "nvfp4_probe.h")
A = 0x7F0000000000          # a 16-byte-aligned fake device address
BIG = 1 << 30               # spacing so fake buffers never overlap


def _declared(path=HDR):
    txt = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(nvfp4_[a-z_0-9]+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(F.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return F.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == set(F.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_probe_library_exports_every_declared_symbol(L):
    from fp4_decode_gemv_amd import probe as P

    names = _declared(PROBE_HDR)
    assert set(names) == set(P.EXPORTED), names
    PL = P.lib()
    for n in names:
        assert hasattr(PL, n), n
    assert P.read_variants()[0].startswith("vgpr_u")


def test_probe_rejects_bad_arguments(L):
    from fp4_decode_gemv_amd import probe as P

    PL = P.lib()
    assert PL.nvfp4_probe_read(-1, A, 1024, 1, A + BIG, None) == -1
    assert PL.nvfp4_probe_read(0, A + 4, 1024, 1, A + BIG, None) == -1   # misaligned
    assert PL.nvfp4_probe_read(0, A, 1000, 1, A + BIG, None) == -1       # not a multiple of 16
    assert PL.nvfp4_probe_read(0, A, 1 << 33, 1, A + BIG, None) == -1    # one slice past 2 GB
    assert PL.nvfp4_probe_convert(9, A, A + BIG, 4, None) == -1
    assert PL.nvfp4_probe_empty(0, 64, None) == -1


def test_noalloc_rejects_shapes_before_any_hip_call(L):
    """The scratch entry point refuses out-of-range shapes and shapes whose
    LM-head workspace exceeds its static array on the host (no GPU here)."""
    assert L.nvfp4_gemv_noalloc_scratch_bytes() == 16 << 20
    e = ctypes.byref(F.LmheadEpilogue(0.6, 0.4, 1.0, 0.6, 8, 0, A, A, A, A))
    args = (A, A + BIG, A + 2 * BIG, A + 3 * BIG, A + 4 * BIG, A + 5 * BIG, A + 6 * BIG)
    assert L.nvfp4_gemv_smallm_noalloc(0, 64, 64, *args, None, None) == F.NVFP4_ERR_SHAPE
    assert F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, 128, 400000, 32) > 16 << 20
    assert L.nvfp4_gemv_smallm_noalloc(128, 400000, 32, *args, e, None) == F.NVFP4_ERR_WORKSPACE


def test_status_strings(L):
    for s in range(0, -8, -1):
        txt = F.status_str(s)
        assert txt.startswith("NVFP4_"), txt
    assert "unknown" in F.status_str(-99)


def _gemv(L, M=1, N=64, K=64, a=A, asc=A + BIG, ag=A + 2 * BIG, w=A + 3 * BIG, wsc=A + 4 * BIG,
          wg=A + 5 * BIG, y=A + 6 * BIG, epi=None, ws=None, wsb=0):
    return L.nvfp4_gemv_smallm(M, N, K, a, asc, ag, w, wsc, wg, y, epi, ws, wsb, None)


def test_gemv_shape_errors(L):
    for M, N, K in [(0, 64, 64), (129, 64, 64), (1, 0, 64), (1, 64, 16), (1, 64, 48), (1, 64, 0), (-1, 64, 64)]:
        assert _gemv(L, M, N, K) == F.NVFP4_ERR_SHAPE, (M, N, K)


def test_gemv_null_align_overlap_errors(L):
    assert _gemv(L, a=None) == F.NVFP4_ERR_NULL
    assert _gemv(L, wg=None) == F.NVFP4_ERR_NULL
    assert _gemv(L, y=None) == F.NVFP4_ERR_NULL
    assert _gemv(L, w=A + 3 * BIG + 8) == F.NVFP4_ERR_ALIGN
    assert _gemv(L, y=A + 6 * BIG + 4) == F.NVFP4_ERR_ALIGN
    # y overlapping the weight codes
    assert _gemv(L, y=A + 3 * BIG + 16) == F.NVFP4_ERR_ARG


def test_gemv_epilogue_errors(L):
    st, ent, tmp, flags = A + 7 * BIG, A + 8 * BIG, A + 9 * BIG, A + 10 * BIG
    def epi(window=8, mode=0, state=st):
        return ctypes.byref(F.LmheadEpilogue(0.6, 0.4, 1.0, 0.6, window, mode, flags, state, ent, tmp))
    need = L.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, 1, 64, 64)
    assert need > 0
    ws = A + 11 * BIG
    assert _gemv(L, epi=epi(window=0), ws=ws, wsb=need) == F.NVFP4_ERR_ARG
    assert _gemv(L, epi=epi(window=2000), ws=ws, wsb=need) == F.NVFP4_ERR_ARG
    assert _gemv(L, epi=epi(mode=3), ws=ws, wsb=need) == F.NVFP4_ERR_ARG
    assert _gemv(L, epi=epi(state=None), ws=ws, wsb=need) == F.NVFP4_ERR_NULL
    assert _gemv(L, epi=epi(state=st + 4), ws=ws, wsb=need) == F.NVFP4_ERR_ALIGN
    assert _gemv(L, epi=epi(), ws=ws, wsb=need - 1) == F.NVFP4_ERR_WORKSPACE
    assert _gemv(L, epi=epi(), ws=None, wsb=need) == F.NVFP4_ERR_WORKSPACE
    # workspace overlapping the logits
    assert _gemv(L, epi=epi(), ws=A + 6 * BIG, wsb=need) == F.NVFP4_ERR_ARG


def test_quantize_act_errors(L):
    q = L.nvfp4_quantize_act
    x, c, s, g = A, A + BIG, A + 2 * BIG, A + 3 * BIG
    assert q(x, 0, 64, c, s, g, 0, None, 0, None) == F.NVFP4_ERR_SHAPE
    assert q(x, 129, 64, c, s, g, 0, None, 0, None) == F.NVFP4_ERR_SHAPE
    assert q(x, 1, 40, c, s, g, 0, None, 0, None) == F.NVFP4_ERR_SHAPE
    assert q(None, 1, 64, c, s, g, 0, None, 0, None) == F.NVFP4_ERR_NULL
    assert q(x, 1, 64, c, s, None, 0, None, 0, None) == F.NVFP4_ERR_NULL
    assert q(x, 1, 64, c, s, g, 7, None, 0, None) == F.NVFP4_ERR_ARG
    assert q(x + 2, 1, 64, c, s, g, 0, None, 0, None) == F.NVFP4_ERR_ALIGN
    assert q(x, 1, 64, x + 16, s, g, 0, None, 0, None) == F.NVFP4_ERR_ARG   # codes inside x
    # large dynamic tensors need the amax workspace
    need = L.nvfp4_workspace_size(F.NVFP4_OP_QUANT, 8, 0, 25600)
    assert need > 0
    assert q(x, 8, 25600, c, s, g, 0, None, 0, None) == F.NVFP4_ERR_WORKSPACE
    assert q(x, 8, 25600, c, s, g, 0, A + 5 * BIG, need - 4, None) == F.NVFP4_ERR_WORKSPACE
    # static scale needs no workspace: passes validation, then fails only at the device check
    assert L.nvfp4_workspace_size(F.NVFP4_OP_QUANT, 1, 0, 4096) == 0


def test_per_token_scale_errors(L):
    q = L.nvfp4_quantize_act
    x, c, s, g = A, A + BIG, A + 2 * BIG, A + 3 * BIG
    assert q(x, 1, 64, c, s, g, 4, None, 0, None) == F.NVFP4_ERR_ARG                 # unknown flag
    assert q(x, 2, 131072 + 32, c, s, g, F.NVFP4_GS_TOKEN_DYNAMIC, None, 0, None) == F.NVFP4_ERR_SHAPE
    # gscale [M]: 8 floats from 4 bytes below the codes reach into them
    assert q(x, 8, 64, c, s, c - 4, F.NVFP4_GS_TOKEN_DYNAMIC, None, 0, None) == F.NVFP4_ERR_ARG
    assert q(x, 8, 64, c, s, c - 4, F.NVFP4_GS_DYNAMIC, None, 0, None) not in (F.NVFP4_ERR_ARG,)
    # per-token flags need no workspace at any size: validation passes
    for fl in (F.NVFP4_GS_TOKEN_DYNAMIC, F.NVFP4_GS_TOKEN_STATIC):
        assert q(x, 8, 25600, c, s, g, fl, None, 0, None) in (F.NVFP4_ERR_DEVICE, F.NVFP4_ERR_HIP)
    gt = L.nvfp4_gemv_smallm_token_scales
    a, asc, ag, w, wsc, wg, y = A, A + BIG, A + 2 * BIG, A + 3 * BIG, A + 4 * BIG, A + 5 * BIG, A + 6 * BIG
    assert gt(0, 64, 64, a, asc, ag, w, wsc, wg, y, None, None, 0, None) == F.NVFP4_ERR_SHAPE
    assert gt(4, 64, 64, a, asc, None, w, wsc, wg, y, None, None, 0, None) == F.NVFP4_ERR_NULL
    # a_gscale [4] reaching into y (its last float is y's first)
    assert gt(4, 64, 64, a, asc, y - 12, w, wsc, wg, y, None, None, 0, None) == F.NVFP4_ERR_ARG
    assert _gemv(L, M=4, ag=y - 12) != F.NVFP4_ERR_ARG    # one scale (4 bytes) ends before y
    assert gt(4, 64, 64, a, asc, ag, w, wsc, wg, y, None, None, 0, None) in (F.NVFP4_ERR_DEVICE, F.NVFP4_ERR_HIP)


def test_pack_errors(L):
    p = L.nvfp4_pack_weights
    w, c, s, g, ws = A, A + BIG, A + 2 * BIG, A + 3 * BIG, A + 4 * BIG
    need = L.nvfp4_workspace_size(F.NVFP4_OP_PACK, 0, 100, 64)
    assert need >= 4
    assert p(w, 0, 64, c, s, g, ws, need, None) == F.NVFP4_ERR_SHAPE
    assert p(w, 100, 20, c, s, g, ws, need, None) == F.NVFP4_ERR_SHAPE
    assert p(None, 100, 64, c, s, g, ws, need, None) == F.NVFP4_ERR_NULL
    assert p(w, 100, 64, c, s, g, None, need, None) == F.NVFP4_ERR_WORKSPACE
    assert p(w, 100, 64, c, s, g, ws, need - 1, None) == F.NVFP4_ERR_WORKSPACE
    assert p(w, 100, 64, c + 1, s, g, ws, need, None) == F.NVFP4_ERR_ALIGN
    assert p(w, 100, 64, w + 64, s, g, ws, need, None) == F.NVFP4_ERR_ARG


def test_reset_state_and_workspace_helpers(L):
    assert L.nvfp4_reset_state_size(0) == 0
    assert L.nvfp4_reset_state_size(2000) == 0
    for w in (1, 8, 32, 1024):
        sz = L.nvfp4_reset_state_size(w)
        assert sz % 16 == 0 and sz >= 4 * w + 32
    assert L.nvfp4_reset_state_init(A, 0, 8, None) == F.NVFP4_ERR_SHAPE
    assert L.nvfp4_reset_state_init(A, 129, 8, None) == F.NVFP4_ERR_SHAPE
    assert L.nvfp4_reset_state_init(A, 1, 0, None) == F.NVFP4_ERR_ARG
    assert L.nvfp4_reset_state_init(None, 1, 8, None) == F.NVFP4_ERR_NULL
    assert L.nvfp4_reset_state_init(A + 8, 1, 8, None) == F.NVFP4_ERR_ALIGN
    assert L.nvfp4_workspace_init(None, 16, None) == F.NVFP4_ERR_NULL
    assert L.nvfp4_workspace_init(A + 4, 16, None) == F.NVFP4_ERR_ALIGN
    assert L.nvfp4_workspace_init(A, 20, None) == F.NVFP4_ERR_ARG
    assert L.nvfp4_workspace_size(F.NVFP4_OP_GEMV, 1, 4096, 4096) == 0
    assert L.nvfp4_workspace_size(99, 1, 4096, 4096) == 0
    # the LM-head workspace grows with N
    a = L.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, 8, 151936, 5120)
    b = L.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, 8, 4096, 5120)
    assert a > b > 0


def test_launch_table_names_real_variants(L):
    """Every shape of the workloads resolves to a compiled variant whose
    token count covers M and whose K granularity K satisfies (host logic
    only: no kernel runs)."""
    import workloads as W

    F.nvfp4_gemv_tune(None, True)
    names = set(F.nvfp4_gemv_variant_names())
    shapes = [(c.N, c.K) for c in W.qwen3_8b_cases() + W.qwen3_32b_cases()]
    shapes += [(W.lm_head_case().N, W.lm_head_case().K), (4096, 4096), (4097, 4128), (300, 96), (1, 32)]
    for (N, K) in shapes:
        for M in range(1, 129):
            for lm in (False, True):
                v = F.nvfp4_gemv_variant(M, N, K, lm)
                assert v in names, (M, N, K, v)
                assert F.variant_tokens(v) >= M, (M, N, K, v)
                assert K % F.variant_k_multiple(v) == 0, (M, N, K, v)


# The launch table's measured choices on the workloads' shapes (host logic
# only).  The eight-token kernel's row groups R follow the rule written in
# default_variant: 40-row tiles balanced over 256 CUs below N = 16384 (qkv:
# 40 rows -> R = 5; o, down: 20 rows -> R = 3 with 8 waves on K >= 8192;
# 4096 rows: 16 -> R = 2), the fewest rows per CU at 16384 <= N < 65536
# (gate_up 51200: R = 5 in 5 rounds; Qwen3-8B gate_up 24576: R = 3 and 4 tie
# at 12, the smaller wins), R = 4 for LM heads.  At 9..16 tokens the
# two-set form is taken only where R comes out at 4 or 5.
LAUNCH_CHOICES = [
    (8, 10240, 5120, False, "stream8_m8_r5_w4_u2"), (8, 5120, 8192, False, "stream8_m8_r3_w8_u2"),
    (8, 51200, 5120, False, "stream8_m8_r5_w4_u2"), (8, 5120, 25600, False, "stream8_m8_r3_w8_u2"),
    (8, 24576, 4096, False, "stream8_m8_r3_w4_u2"), (8, 4096, 4096, False, "stream8_m8_r2_w4_u2"),
    (8, 4096, 12288, False, "stream8_m8_r2_w8_u2"), (8, 151936, 5120, True, "stream8_m8_r4_w4_u2"),
    (5, 151936, 5120, False, "stream8_m8_r4_w4_u2"), (2, 51200, 5120, False, "stream8_m8_r5_w4_u2"),
    (4, 5120, 8192, False, "stream_m4_r5_w4_u2"), (2, 5120, 25600, False, "stream8_m8_r3_w8_u2"),
    (4, 4096, 12288, False, "stream8_m8_r2_w8_u2"), (1, 4096, 12288, False, "stream8_m8_r2_w8_u2"),
    (1, 5120, 8192, False, "direct_m1_g64_r1_w4_p1_nt"), (1, 5120, 25600, False, "direct_m1_g64_r1_w4_p1_nt"),
    (1, 6144, 4096, False, "stream8_m8_r3_w4_u2"),
    (2, 151936, 5120, False, "wstream_m4_r3_w4_u2_ag"), (4, 151936, 5120, False, "wstream_m4_r3_w4_u2"),
    (1, 4096, 4096, False, "stream8_m8_r2_w4_u2"), (1, 10240, 5120, False, "direct_m1_g32_r1_w4_p1_nt"),
    (1, 51200, 5120, False, "staged_m1_g32_r2_w4_p1"), (1, 151936, 5120, True, "direct_m1_g32_r2_w4_p1_nt"),
    (1, 151936, 5120, False, "direct_m1_g32_r2_w4_p1_nt"),
    (8, 1024, 4128, False, "lmfma_m8_r1_w4_p1"),
    (16, 10240, 5120, False, "stream8_m16_r5_w4_u2"), (12, 51200, 5120, False, "stream8_m16_r5_w4_u2"),
    (16, 151936, 5120, True, "stream8_m16_r4_w4_u2"), (16, 5120, 8192, False, "lmfma_m16_r2_w8_p1"),
    (16, 24576, 4096, False, "lmfma_m16_r2_w4_p1"), (9, 4096, 4096, False, "lmfma_m16_r2_w4_p1"),
    # 17..128 tokens: the tiled GEMM on gate_up (many row tiles) and, split
    # along K, on down at 65..128; the register-staged kernel elsewhere (the
    # split GEMM measured slower on qkv, o and down at 24..64 tokens)
    (32, 51200, 5120, False, "gemm_m32"), (64, 51200, 5120, False, "gemm_m64"),
    (128, 51200, 5120, False, "gemm_m128"), (128, 5120, 25600, False, "gemm_m128"),
    (32, 10240, 5120, False, "lmfma_m32_r2_w4_p1"), (64, 10240, 5120, False, "lmfma_m64_r2_w4_p1"),
    (128, 10240, 5120, False, "lmfma_m128_r2_w4_p1"), (32, 5120, 8192, False, "lmfma_m32_r2_w8_p1"),
    (64, 5120, 8192, False, "lmfma_m64_r2_w4_p1"), (32, 5120, 25600, False, "lmfma_m32_r2_w8_p1"),
    (64, 5120, 25600, False, "lmfma_m64_r2_w8_p1"),
]


@pytest.mark.parametrize("M,N,K,lm,variant", LAUNCH_CHOICES)
def test_launch_choices_on_the_workload_shapes(L, M, N, K, lm, variant):
    F.nvfp4_gemv_tune(None, True)
    assert F.nvfp4_gemv_variant(M, N, K, lm) == variant


def test_forced_variant_falls_back_when_k_does_not_fit(L):
    """A direct-to-LDS variant forced on a K that is not a multiple of 256
    is not launched; the default for that shape is used instead."""
    with F.forced_variant("dma_m8_r2_w4_d3"):
        assert F.nvfp4_gemv_variant(8, 1024, 4096) == "dma_m8_r2_w4_d3"
        v = F.nvfp4_gemv_variant(8, 1024, 4128)
        assert v != "dma_m8_r2_w4_d3" and 4128 % F.variant_k_multiple(v) == 0
    assert F.nvfp4_gemv_variant(8, 1024, 4096) != "dma_m8_r2_w4_d3"


def test_gemv_tune_rejects_unknown_names(L):
    assert L.nvfp4_gemv_tune(b"no_such_variant", 1) == F.NVFP4_ERR_ARG
    assert L.nvfp4_gemv_tune(None, 2) == F.NVFP4_ERR_ARG
    assert L.nvfp4_gemv_tune(None, 1) == F.NVFP4_OK
    with pytest.raises(F.Nvfp4Error):
        F.nvfp4_gemv_tune("no_such_variant")


def test_quantize_rejects_tensors_past_32_bit_offsets(L):
    """A per-tensor quantization of M x K >= 2^30 elements is a shape error
    (its 2-byte elements are addressed with 32-bit byte offsets); per-token
    rows are short enough."""
    far = 1 << 44
    x, c, sc, g, ws = A, A + far, A + 2 * far, A + 3 * far, A + 4 * far
    assert L.nvfp4_quantize_act(x, 128, 1 << 23, c, sc, g, F.NVFP4_GS_STATIC, ws, 1 << 40, None) == F.NVFP4_ERR_SHAPE
    assert L.nvfp4_quantize_act(x, 128, 1 << 24, c, sc, g, F.NVFP4_GS_DYNAMIC, ws, 1 << 40, None) == F.NVFP4_ERR_SHAPE


def test_gemv_epilogue_partials_beyond_2gb_are_a_shape_error(L):
    """The LM-head merge addresses its per-workgroup partials with 32-bit
    offsets, so an N whose partials would pass 2 GB is rejected before any
    HIP call (fake buffers far apart, never dereferenced)."""
    far = 1 << 44
    st, ent, tmp, flags = A + 7 * far, A + 8 * far, A + 9 * far, A + 10 * far
    e = ctypes.byref(F.LmheadEpilogue(0.6, 0.4, 1.0, 0.6, 8, 0, flags, st, ent, tmp))
    M, N, K = 8, 1 << 32, 32
    assert L.nvfp4_gemv_smallm(M, N, K, A, A + far, A + 2 * far, A + 3 * far, A + 4 * far, A + 5 * far,
                               A + 6 * far, e, A + 11 * far, 1 << 40, None) == F.NVFP4_ERR_SHAPE


def test_sample_top_p_errors(L):
    s = L.nvfp4_sample_top_p
    z, T, u, tok, nuc, ws = A, A + BIG, A + 2 * BIG, A + 3 * BIG, A + 4 * BIG, A + 5 * BIG
    need = L.nvfp4_workspace_size(F.NVFP4_OP_SAMPLE, 2, 100, 0)
    assert need > 0
    assert L.nvfp4_workspace_size(F.NVFP4_OP_SAMPLE, 8, 151936, 0) > L.nvfp4_workspace_size(F.NVFP4_OP_SAMPLE, 1, 151936, 0)
    assert L.nvfp4_workspace_size(F.NVFP4_OP_SAMPLE, 0, 100, 0) == 0

    def call(M=2, N=100, z=z, T=T, p=0.95, u=u, tok=tok, nuc=nuc, ws=ws, wsb=need):
        return s(M, N, z, T, p, u, tok, nuc, ws, wsb, None)

    assert call(M=0) == F.NVFP4_ERR_SHAPE
    assert call(M=65536) == F.NVFP4_ERR_SHAPE
    assert call(N=0) == F.NVFP4_ERR_SHAPE
    assert call(N=1 << 24) == F.NVFP4_ERR_SHAPE
    assert call(z=None) == F.NVFP4_ERR_NULL
    assert call(T=None) == F.NVFP4_ERR_NULL
    assert call(u=None) == F.NVFP4_ERR_NULL
    assert call(tok=None) == F.NVFP4_ERR_NULL
    assert call(z=z + 2) == F.NVFP4_ERR_ALIGN
    assert call(tok=tok + 1) == F.NVFP4_ERR_ALIGN
    for p in (0.0, -0.5, 1.0001, float("nan")):
        assert call(p=p) == F.NVFP4_ERR_ARG, p
    assert call(ws=None) == F.NVFP4_ERR_WORKSPACE
    assert call(wsb=need - 1) == F.NVFP4_ERR_WORKSPACE
    assert call(ws=ws + 8) == F.NVFP4_ERR_ALIGN
    assert call(tok=z + 40) == F.NVFP4_ERR_ARG        # tokens inside the logits
    assert call(nuc=tok + 4) == F.NVFP4_ERR_ARG       # nucleus overlapping tokens
    assert call(tok=T) == F.NVFP4_ERR_ARG             # output over an input
    assert call(ws=z + 256) == F.NVFP4_ERR_ARG        # workspace over the logits
    assert call(ws=tok - 256) == F.NVFP4_ERR_ARG      # workspace over an output


def test_quantize_rotated_rejects_bad_arguments(L):
    """Q+R: rotation sizes other than 16/32/64/128 and per-token flags are
    argument errors, K not a multiple of the rotation a shape error, all
    before any HIP call."""
    far = 1 << 44
    x, c, sc, g, ws = A, A + far, A + 2 * far, A + 3 * far, A + 4 * far
    q = L.nvfp4_quantize_act_rotated
    for rot in (0, 8, 48, 256):
        assert q(x, 1, 512, rot, c, sc, g, F.NVFP4_GS_DYNAMIC, ws, 1 << 40, None) == F.NVFP4_ERR_ARG
    for flags in (F.NVFP4_GS_TOKEN_DYNAMIC, F.NVFP4_GS_TOKEN_STATIC, 7):
        assert q(x, 1, 512, 16, c, sc, g, flags, ws, 1 << 40, None) == F.NVFP4_ERR_ARG
    assert q(x, 1, 96, 64, c, sc, g, F.NVFP4_GS_DYNAMIC, ws, 1 << 40, None) == F.NVFP4_ERR_SHAPE
    assert q(x, 1, 160, 128, c, sc, g, F.NVFP4_GS_STATIC, ws, 1 << 40, None) == F.NVFP4_ERR_SHAPE
    assert q(x, 0, 512, 16, c, sc, g, F.NVFP4_GS_STATIC, ws, 1 << 40, None) == F.NVFP4_ERR_SHAPE
    assert q(x, 128, 1 << 23, 16, c, sc, g, F.NVFP4_GS_STATIC, ws, 1 << 40, None) == F.NVFP4_ERR_SHAPE
    assert q(None, 1, 512, 16, c, sc, g, F.NVFP4_GS_STATIC, ws, 1 << 40, None) == F.NVFP4_ERR_NULL
    assert q(x + 8, 1, 512, 16, c, sc, g, F.NVFP4_GS_STATIC, ws, 1 << 40, None) == F.NVFP4_ERR_ALIGN
    # the two-launch dynamic path needs its partials workspace
    assert q(x, 8, 25600, 16, c, sc, g, F.NVFP4_GS_DYNAMIC, None, 0, None) == F.NVFP4_ERR_WORKSPACE
    # overlapping output and input
    assert q(x, 1, 512, 16, x, sc, g, F.NVFP4_GS_STATIC, ws, 1 << 40, None) == F.NVFP4_ERR_ARG


def test_rotated_quantization_workspace_sizes(L):
    """Q+R keeps one launch up to 32768 elements at rot = 16 (halved per
    doubling of rot) and needs amax partials above; unknown rotations ask
    for nothing (the call itself rejects them)."""
    ws = lambda M, rot, K: L.nvfp4_workspace_size(F.NVFP4_OP_QUANT_ROTATED, M, rot, K)
    assert ws(1, 16, 32768) == 0 and ws(2, 16, 32768) > 0
    assert ws(1, 32, 16384) == 0 and ws(1, 32, 16896) > 0
    assert ws(1, 128, 4096) == 0 and ws(1, 128, 5120) > 0
    assert ws(8, 16, 25600) == L.nvfp4_workspace_size(F.NVFP4_OP_QUANT, 8, 0, 25600)
    assert ws(1, 48, 4096) == 0 and ws(0, 16, 4096) == 0
