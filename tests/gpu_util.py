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


def oracle_rows_ref(w: np.ndarray, s_g, a_qs, chunk: int = 2048, workers: int = 8):
    """The oracle's (y, ref_abs) for every row of a large weight matrix w
    (fp32 [N][K], global scale s_g of the whole matrix) against each of the
    oracle's quantized activations in a_qs: the oracle's own quantization
    (once per row chunk) and fp64 GEMV, run on row chunks in threads (numpy
    releases the GIL), joined in row order."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import nvfp4_oracle as O

    N = w.shape[0]
    starts = list(range(0, N, chunk))

    def one(r0):
        wq = O.quantize_nvfp4(w[r0:r0 + chunk], s_g)
        return [O.gemv_ref(a_q, wq) for a_q in a_qs]

    with ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(one, starts))
    return [(np.concatenate([p[i][0] for p in parts], axis=1), np.concatenate([p[i][1] for p in parts], axis=1))
            for i in range(len(a_qs))]
