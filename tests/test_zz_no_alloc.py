"""The GEMV entry point that allocates nothing (its LM-head workspace is the
library's static per-GPU scratch array), called through the C ABI, against
nvfp4_gemv_smallm with a caller workspace on the same inputs: identical
outputs (the same kernels run), entropies and temperatures, and both within
the oracle's tolerance.  Two calls in a row, the second with a smaller
input, so the scratch's leftover contents of the first must not matter."""

import ctypes

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
import workloads as W
from oracle import nvfp4_oracle as O
from oracle import reset_oracle as R
from gpu_util import assert_gemv_close, bf16_dev, f32_dev

pytestmark = pytest.mark.gpu


def _ptr(t):
    return int(t.data_ptr())


def _case(M, N, K, seed):
    w = W.small_random_weights(seed, N, K, scale=0.2)
    xb = W.small_random_bf16(seed + 1, M, K)
    return w, xb, F.nvfp4_pack_weights(f32_dev(w)), F.nvfp4_quantize_act(bf16_dev(xb))


def _epi(M, dev):
    return F.Epilogue(step_start=torch.ones(M, dtype=torch.uint8, device=dev), state=F.new_reset_state(M, 8, dev),
                      entropy=torch.empty(M, device=dev), temperature=torch.empty(M, device=dev))


@pytest.mark.parametrize("with_epilogue", [True, False])
def test_noalloc_matches_workspace_entry_point(with_epilogue):
    L = F.lib()
    dev = torch.device("cuda:0")
    for (M, N, K, seed) in ((8, 40000, 1024, 61), (2, 5000, 512, 62)):  # second call smaller
        print(f"[noalloc] epilogue={with_epilogue} M={M} N={N} K={K}", flush=True)
        w, xb, wq, aq = _case(M, N, K, seed)
        # reference: the existing entry point with a caller workspace
        e_ref = _epi(M, dev) if with_epilogue else None
        y_ref = F.nvfp4_gemv_smallm(aq, wq, epi=e_ref)
        # the scratch entry point, straight through the C ABI
        y = torch.full((M, N), float("nan"), device=dev)
        e = _epi(M, dev) if with_epilogue else None
        ce = None if e is None else ctypes.byref(e.as_c())
        st = L.nvfp4_gemv_smallm_noalloc(M, N, K, _ptr(aq.codes), _ptr(aq.scales), _ptr(aq.gscale), _ptr(wq.codes),
                                         _ptr(wq.scales), _ptr(wq.gscale), _ptr(y), ce,
                                         int(torch.cuda.current_stream().cuda_stream) or None)
        assert st == F.NVFP4_OK, F.status_str(st)
        torch.cuda.synchronize()
        yg = y.cpu().numpy()
        assert np.array_equal(yg, y_ref.cpu().numpy())
        ref, ref_abs = O.gemv_ref(O.quantize_act_bf16(xb), O.quantize_nvfp4(w))
        assert_gemv_close(yg, ref, ref_abs, what=f"noalloc M={M} N={N} K={K}")
        if with_epilogue:
            H = e.entropy.cpu().numpy()
            assert np.array_equal(H, e_ref.entropy.cpu().numpy())
            assert np.array_equal(e.temperature.cpu().numpy(), e_ref.temperature.cpu().numpy())
            assert np.all(np.abs(H - R.entropy_rows(yg.astype(np.float64))) <= 1e-4)


def _noalloc(aq, wq, M, N, K):
    y = torch.full((M, N), float("nan"), device="cuda:0")
    st = F.lib().nvfp4_gemv_smallm_noalloc(M, N, K, _ptr(aq.codes), _ptr(aq.scales), _ptr(aq.gscale),
                                           _ptr(wq.codes), _ptr(wq.scales), _ptr(wq.gscale), _ptr(y), None,
                                           int(torch.cuda.current_stream().cuda_stream) or None)
    assert st == F.NVFP4_OK, F.status_str(st)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_noalloc_split_gemm_partials_in_scratch():
    """65..128 tokens on long K: the K-split GEMM keeps its partial sums in
    the scratch array; the same kernels as with a caller workspace, so the
    outputs are identical.  The second, smaller call reuses the scratch."""
    for (M, N, K, seed) in ((128, 1000, 16384, 71), (65, 777, 16640, 72)):
        print(f"[noalloc split] M={M} N={N} K={K}", flush=True)
        assert F.nvfp4_gemv_variant(M, N, K) == "gemm_m128"
        ws = F.nvfp4_workspace_size(F.NVFP4_OP_GEMV, M, N, K)
        assert 0 < ws <= F.lib().nvfp4_gemv_noalloc_scratch_bytes()
        w, xb, wq, aq = _case(M, N, K, seed)
        y_ref = F.nvfp4_gemv_smallm(aq, wq).cpu().numpy()
        yg = _noalloc(aq, wq, M, N, K)
        assert np.array_equal(yg, y_ref)
        ref, ref_abs = O.gemv_ref(O.quantize_act_bf16(xb), O.quantize_nvfp4(w))
        assert_gemv_close(yg, ref, ref_abs, what=f"noalloc split M={M} N={N} K={K}")


def test_noalloc_without_room_for_the_split_uses_another_kernel():
    """A shape whose full K split would not fit the scratch array is not
    refused: the launch table picks a kernel without partial sums there."""
    M, N, K = 128, 2560, 16384
    assert F.nvfp4_gemv_variant(M, N, K) == "gemm_m128"
    assert F.nvfp4_workspace_size(F.NVFP4_OP_GEMV, M, N, K) > F.lib().nvfp4_gemv_noalloc_scratch_bytes()
    print(f"[noalloc no-split] M={M} N={N} K={K}", flush=True)
    w, xb, wq, aq = _case(M, N, K, 73)
    yg = _noalloc(aq, wq, M, N, K)
    ref, ref_abs = O.gemv_ref(O.quantize_act_bf16(xb), O.quantize_nvfp4(w))
    assert_gemv_close(yg, ref, ref_abs, what=f"noalloc fallback M={M} N={N} K={K}")
    assert_gemv_close(F.nvfp4_gemv_smallm(aq, wq).cpu().numpy(), ref, ref_abs, what="workspace entry")


def test_noalloc_rejects_workspace_beyond_scratch():
    """A shape whose LM-head workspace exceeds the scratch array is refused
    before any launch; the output is untouched."""
    L = F.lib()
    dev = torch.device("cuda:0")
    M, N, K = 128, 400000, 32
    assert F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, M, N, K) > L.nvfp4_gemv_noalloc_scratch_bytes()
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)
    y = torch.full((4,), 7.0, device=dev)
    e = F.LmheadEpilogue(0.6, 0.4, 1.0, 0.6, 8, 0, _ptr(buf), _ptr(buf), _ptr(buf), _ptr(buf))
    st = L.nvfp4_gemv_smallm_noalloc(M, N, K, _ptr(buf), _ptr(buf), _ptr(buf), _ptr(buf), _ptr(buf), _ptr(buf),
                                     _ptr(y), ctypes.byref(e), None)
    assert st == F.NVFP4_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
