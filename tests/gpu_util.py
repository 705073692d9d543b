"""Helpers shared by the GPU parity tests (device transfer only; no method
arithmetic here)."""

import numpy as np
import torch

import fp4_decode_gemv_amd as F


def dev():
    return torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> contiguous bfloat16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(dev()).view(torch.bfloat16).contiguous()


def f32_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


def host(q: F.NvFp4Tensor):
    torch.cuda.synchronize()
    return q.codes.cpu().numpy(), q.scales.cpu().numpy(), np.float32(q.gscale.cpu().numpy()[0])


def assert_same_q(got, ref, rows=None, what=""):
    gc, gs, gg = got
    rc, rs, rg = ref
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert gg.view(np.uint32) == np.float32(rg).view(np.uint32), (what, gg, rg)
    bad = np.nonzero(gc != rc)
    assert bad[0].size == 0, (what, "codes differ at", bad[0][:5], bad[1][:5])
    bad = np.nonzero(gs != rs)
    assert bad[0].size == 0, (what, "scales differ at", bad[0][:5], bad[1][:5])


def assert_gemv_close(y_gpu: np.ndarray, y_ref: np.ndarray, ref_abs: np.ndarray, what="", tol=1e-5):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = tol * ref_abs
    ok = err <= bound
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} outputs out of tolerance; first at {tuple(i)}: "
                             f"gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r} ref_abs={ref_abs[tuple(i)]!r}")
    return float(np.max(err / np.maximum(ref_abs, 1e-300)))
