"""ctypes binding of ``lib/libnvfp4_probe.so`` (``include/nvfp4_probe.h``):
the HBM read-stream probe and the converter probe.  Measurement and test
tools only; the projection library never calls them.  Argument marshalling
only: the reads and conversions run in the library's HIP kernels."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "lib", "libnvfp4_probe.so")

FP4_TO_F16 = 0
FP4_TO_F32 = 1
FP8_TO_F32 = 2
F32_TO_FP4 = 3
F16_SCALE_MUL = 4

EXPORTED = ("nvfp4_probe_read_count", "nvfp4_probe_read_name", "nvfp4_probe_read", "nvfp4_probe_empty",
            "nvfp4_probe_convert")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(f"probe library not built ({PROBE_LIB_PATH} missing)")
    L = ctypes.CDLL(PROBE_LIB_PATH)
    vp, sz, c_int = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.nvfp4_probe_read_count.restype = c_int
    L.nvfp4_probe_read_count.argtypes = []
    L.nvfp4_probe_read_name.restype = ctypes.c_char_p
    L.nvfp4_probe_read_name.argtypes = [c_int]
    L.nvfp4_probe_read.restype = c_int
    L.nvfp4_probe_read.argtypes = [c_int, vp, sz, c_int, vp, vp]
    L.nvfp4_probe_empty.restype = c_int
    L.nvfp4_probe_empty.argtypes = [c_int, c_int, vp]
    L.nvfp4_probe_convert.restype = c_int
    L.nvfp4_probe_convert.argtypes = [c_int, vp, vp, c_int, vp]
    _lib = L
    return L


def _stream(stream) -> int | None:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) or None


def read_variants() -> list[str]:
    L = lib()
    return [L.nvfp4_probe_read_name(i).decode() for i in range(L.nvfp4_probe_read_count())]


def read(variant: int, buf, nbytes: int, grid: int, sink, stream=None) -> None:
    """One probe read of the first ``nbytes`` bytes of device tensor ``buf``."""
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if sink.numel() * sink.element_size() < 4 * grid:
        raise ValueError("sink needs one uint32 per workgroup")
    st = lib().nvfp4_probe_read(int(variant), buf.data_ptr(), int(nbytes), int(grid), sink.data_ptr(),
                                _stream(stream))
    if st != 0:
        raise RuntimeError(f"nvfp4_probe_read failed: status {st}")


def empty(grid: int, threads: int = 256, stream=None) -> None:
    st = lib().nvfp4_probe_empty(int(grid), int(threads), _stream(stream))
    if st != 0:
        raise RuntimeError(f"nvfp4_probe_empty failed: status {st}")


_OUT_PER_IN = {FP4_TO_F16: 4, FP4_TO_F32: 8, FP8_TO_F32: 4, F32_TO_FP4: 1, F16_SCALE_MUL: 1}
_IN_PER_ITEM = {FP4_TO_F16: 1, FP4_TO_F32: 1, FP8_TO_F32: 1, F32_TO_FP4: 2, F16_SCALE_MUL: 2}


def convert(op: int, words):
    """Run converter ``op`` on a host uint32 numpy array; returns the uint32
    outputs as a numpy array (layouts in include/nvfp4_probe.h)."""
    import numpy as np
    import torch

    words = np.ascontiguousarray(words, dtype=np.uint32)
    if words.size % _IN_PER_ITEM[op] != 0:
        raise ValueError("two-operand converters take pairs")
    n = words.size // _IN_PER_ITEM[op]
    d_in = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    d_out = torch.zeros(n * _OUT_PER_IN[op], dtype=torch.int32, device="cuda:0")
    st = lib().nvfp4_probe_convert(int(op), d_in.data_ptr(), d_out.data_ptr(), int(n), _stream(None))
    if st != 0:
        raise RuntimeError(f"nvfp4_probe_convert failed: status {st}")
    torch.cuda.synchronize()
    return d_out.cpu().numpy().view(np.uint32)
