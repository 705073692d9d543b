"""CPU tests of the Python binding's argument checks: the C ABI sees only
pointers, so the wrappers reject every size, dtype, layout and device
mismatch with ValueError before any library call (CPU tensors, no GPU)."""

import pytest
import torch

import fp4_decode_gemv_amd as F


def nv(rows, K, gs=1):
    return F.NvFp4Tensor(torch.zeros((rows, K // 2), dtype=torch.uint8), torch.zeros((rows, K // 16), dtype=torch.uint8),
                         torch.ones(gs, dtype=torch.float32))


def test_gemv_rejects_mismatched_k():
    with pytest.raises(ValueError, match="K"):
        F.nvfp4_gemv_smallm(nv(2, 64), nv(8, 128))


def test_gemv_rejects_m_beyond_activation_rows():
    with pytest.raises(ValueError, match="M must be"):
        F.nvfp4_gemv_smallm(nv(2, 64), nv(8, 64), M=3)


def test_gemv_rejects_bad_output():
    a, w = nv(2, 64), nv(8, 64)
    with pytest.raises(ValueError, match="shape"):
        F.nvfp4_gemv_smallm(a, w, y=torch.empty((2, 7)))
    with pytest.raises(ValueError, match="float32"):
        F.nvfp4_gemv_smallm(a, w, y=torch.empty((2, 8), dtype=torch.float64))
    with pytest.raises(ValueError, match="contiguous"):
        F.nvfp4_gemv_smallm(a, w, y=torch.empty((8, 2)).t())


def test_gemv_rejects_bad_scales_and_codes():
    a, w = nv(2, 64), nv(8, 64)
    w.scales = torch.zeros((8, 3), dtype=torch.uint8)
    with pytest.raises(ValueError, match="w.scales"):
        F.nvfp4_gemv_smallm(a, w)
    a, w = nv(2, 64), nv(8, 64)
    a.codes = a.codes.to(torch.int8)
    with pytest.raises(ValueError, match="a.codes"):
        F.nvfp4_gemv_smallm(a, w)


def test_gemv_rejects_short_per_token_scales():
    a, w = nv(4, 64, gs=2), nv(8, 64)
    with pytest.raises(ValueError, match="per-token"):
        F.nvfp4_gemv_smallm(a, w)


def test_gemv_rejects_short_epilogue_buffers():
    a, w = nv(4, 64), nv(8, 64)
    epi = F.Epilogue(step_start=torch.zeros(3, dtype=torch.uint8), state=torch.zeros(4096, dtype=torch.uint8),
                     entropy=torch.zeros(4), temperature=torch.zeros(4))
    with pytest.raises(ValueError, match="step_start"):
        F.nvfp4_gemv_smallm(a, w, epi=epi)


def test_pack_rejects_bad_weights():
    with pytest.raises(ValueError, match="float32"):
        F.nvfp4_pack_weights(torch.zeros((4, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        F.nvfp4_pack_weights(torch.zeros((64, 4)).t())
    with pytest.raises(ValueError, match="out.codes"):
        F.nvfp4_pack_weights(torch.zeros((4, 64)), out=nv(4, 32))
    bad = nv(4, 64)
    bad.scales = torch.zeros((4, 5), dtype=torch.uint8)
    with pytest.raises(ValueError, match="out.scales"):
        F.nvfp4_pack_weights(torch.zeros((4, 64)), out=bad)


def test_quantize_rejects_bad_inputs():
    with pytest.raises(ValueError, match="bfloat16"):
        F.nvfp4_quantize_act(torch.zeros((2, 64)))
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="gscale"):
        F.nvfp4_quantize_act(x, gscale=torch.ones(2), per_token=True)
    with pytest.raises(ValueError, match="out.codes"):
        F.nvfp4_quantize_act(x, out=nv(2, 64))


def test_every_wrapper_that_uses_torch_imports_it():
    """The binding imports torch inside each function (the module loads
    without it); a wrapper that forgot would fail only on the path that
    first touches torch, e.g. allocating a workspace the caller did not
    pass."""
    import ast
    import inspect

    tree = ast.parse(inspect.getsource(F))
    missing = []
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            uses = any(isinstance(n, ast.Name) and n.id == "torch" for n in ast.walk(fn))
            imports = any(isinstance(n, ast.Import) and any(a.name == "torch" for a in n.names) for n in ast.walk(fn))
            if uses and not imports:
                missing.append(fn.name)
    assert not missing, missing
