"""Python binding of the gfx950 NVFP4 small-M decode-projection library.

A thin ctypes layer over ``lib/libnvfp4.so`` (the C ABI in
``include/nvfp4.h``).  It only marshals arguments: torch tensors supply
device memory (``data_ptr()``) and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or fails to load, every call raises.

Functions keep the C names:

* ``nvfp4_pack_weights(w)`` -> ``(codes, scales, gscale)``
* ``nvfp4_quantize_act(x_bf16, gscale=None)`` -> ``(codes, scales, gscale)``
* ``nvfp4_quantize_act_rotated(x_bf16, rot=16, gscale=None)`` -> the same,
  after a block Walsh-Hadamard rotation of each row ("Q+R")
* ``nvfp4_gemv_smallm(a, w, ...)`` -> ``y`` (optionally with the LM-head
  epilogue)
* ``nvfp4_sample_top_p(logits, temperature, top_p, uniforms)`` ->
  ``(tokens, nucleus)``
* ``nvfp4_workspace_size``, ``nvfp4_workspace_init``,
  ``nvfp4_reset_state_size``, ``nvfp4_reset_state_init``,
  ``nvfp4_status_str``.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libnvfp4.so")

NVFP4_OK = 0
NVFP4_ERR_NULL = -1
NVFP4_ERR_SHAPE = -2
NVFP4_ERR_ALIGN = -3
NVFP4_ERR_WORKSPACE = -4
NVFP4_ERR_DEVICE = -5
NVFP4_ERR_HIP = -6
NVFP4_ERR_ARG = -7

NVFP4_GS_DYNAMIC = 0
NVFP4_GS_STATIC = 1
NVFP4_GS_TOKEN_DYNAMIC = 2
NVFP4_GS_TOKEN_STATIC = 3

NVFP4_OP_PACK = 0
NVFP4_OP_QUANT = 1
NVFP4_OP_GEMV = 2
NVFP4_OP_GEMV_LMHEAD = 3
NVFP4_OP_SAMPLE = 4
NVFP4_OP_QUANT_ROTATED = 5

EXPORTED = (
    "nvfp4_status_str",
    "nvfp4_workspace_size",
    "nvfp4_workspace_init",
    "nvfp4_pack_weights",
    "nvfp4_quantize_act",
    "nvfp4_quantize_act_rotated",
    "nvfp4_reset_state_size",
    "nvfp4_reset_state_init",
    "nvfp4_gemv_smallm",
    "nvfp4_gemv_smallm_token_scales",
    "nvfp4_gemv_smallm_noalloc",
    "nvfp4_gemv_noalloc_scratch_bytes",
    "nvfp4_gemv_variant",
    "nvfp4_gemv_variant_name",
    "nvfp4_gemv_tune",
    "nvfp4_sample_top_p",
)


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


class LmheadEpilogue(ctypes.Structure):
    """Mirror of ``nvfp4_lmhead_epilogue_t``."""

    _fields_ = [
        ("tau0", ctypes.c_float),
        ("t_low", ctypes.c_float),
        ("t_high", ctypes.c_float),
        ("t_base", ctypes.c_float),
        ("window", ctypes.c_int),
        ("mode", ctypes.c_int),
        ("step_start", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("entropy", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not built ({LIB_PATH} missing); run `python -c 'import __graft_entry__ as g; g.build()'`"
        )
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    c_int = ctypes.c_int
    L.nvfp4_status_str.restype = ctypes.c_char_p
    L.nvfp4_status_str.argtypes = [c_int]
    L.nvfp4_workspace_size.restype = sz
    L.nvfp4_workspace_size.argtypes = [c_int, c_int, i64, i64]
    L.nvfp4_workspace_init.restype = c_int
    L.nvfp4_workspace_init.argtypes = [vp, sz, vp]
    L.nvfp4_pack_weights.restype = c_int
    L.nvfp4_pack_weights.argtypes = [vp, i64, i64, vp, vp, vp, vp, sz, vp]
    L.nvfp4_quantize_act.restype = c_int
    L.nvfp4_quantize_act.argtypes = [vp, c_int, i64, vp, vp, vp, c_int, vp, sz, vp]
    L.nvfp4_quantize_act_rotated.restype = c_int
    L.nvfp4_quantize_act_rotated.argtypes = [vp, c_int, i64, c_int, vp, vp, vp, c_int, vp, sz, vp]
    L.nvfp4_reset_state_size.restype = sz
    L.nvfp4_reset_state_size.argtypes = [c_int]
    L.nvfp4_reset_state_init.restype = c_int
    L.nvfp4_reset_state_init.argtypes = [vp, c_int, c_int, vp]
    L.nvfp4_gemv_variant.restype = ctypes.c_char_p
    L.nvfp4_gemv_variant.argtypes = [c_int, i64, i64, c_int]
    L.nvfp4_gemv_variant_name.restype = ctypes.c_char_p
    L.nvfp4_gemv_variant_name.argtypes = [c_int]
    L.nvfp4_gemv_tune.restype = c_int
    L.nvfp4_gemv_tune.argtypes = [ctypes.c_char_p, c_int]
    L.nvfp4_gemv_smallm.restype = c_int
    L.nvfp4_gemv_smallm.argtypes = [c_int, i64, i64, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.POINTER(LmheadEpilogue), vp, sz, vp]
    L.nvfp4_gemv_smallm_token_scales.restype = c_int
    L.nvfp4_gemv_smallm_token_scales.argtypes = L.nvfp4_gemv_smallm.argtypes
    L.nvfp4_gemv_smallm_noalloc.restype = c_int
    L.nvfp4_gemv_smallm_noalloc.argtypes = [c_int, i64, i64, vp, vp, vp, vp, vp, vp, vp,
                                            ctypes.POINTER(LmheadEpilogue), vp]
    L.nvfp4_gemv_noalloc_scratch_bytes.restype = sz
    L.nvfp4_gemv_noalloc_scratch_bytes.argtypes = []
    L.nvfp4_sample_top_p.restype = c_int
    L.nvfp4_sample_top_p.argtypes = [c_int, i64, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().nvfp4_status_str(int(status)).decode()


nvfp4_status_str = status_str


def _check(status: int, where: str) -> None:
    if status != NVFP4_OK:
        raise Nvfp4Error(status, where)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> int | None:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) or None


def _require(t, name: str, dtype, device, shape=None, min_numel: int | None = None) -> None:
    """Raise ValueError unless t is a contiguous tensor of dtype on device
    (with the given shape / at least min_numel elements).  The C ABI sees
    only pointers, so every size it relies on is checked here."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} needs at least {min_numel} elements, got {t.numel()}")


def _require_ws(ws, need: int, device) -> None:
    import torch

    if ws is None:
        return
    _require(ws, "ws", torch.uint8, device)
    if ws.numel() < need:
        raise ValueError(f"ws holds {ws.numel()} bytes, {need} needed")


@dataclass
class NvFp4Tensor:
    """An NVFP4 matrix on the device: codes [rows][K/2], E4M3 scales
    [rows][K/16], global scale [1] (all torch tensors)."""

    codes: "object"
    scales: "object"
    gscale: "object"

    @property
    def rows(self) -> int:
        return int(self.codes.shape[0])

    @property
    def K(self) -> int:
        return int(self.codes.shape[1]) * 2


_WS_SIZES: dict = {}
_TUNING = (None, 1)  # (forced variant, balance) last set through nvfp4_gemv_tune


def nvfp4_workspace_size(op: int, M: int, N: int, K: int) -> int:
    # remembered per shape and per tuning override (which can change it)
    key = (op, M, N, K, _TUNING)
    n = _WS_SIZES.get(key)
    if n is None:
        n = _WS_SIZES[key] = int(lib().nvfp4_workspace_size(op, M, N, K))
    return n


def nvfp4_gemv_tune(variant: str | None = None, balance: bool = True) -> None:
    """Force a compiled GEMV variant for every shape it covers (None: the
    launch table's choice) and choose the MFMA kernels' row mapping
    (balance=False: whole tiles).  Process-wide; for tuning and tests."""
    global _TUNING
    name = None if variant is None else variant.encode()
    _check(lib().nvfp4_gemv_tune(name, int(bool(balance))), "nvfp4_gemv_tune")
    _TUNING = (variant, int(bool(balance)))


class forced_variant:
    """Context manager around nvfp4_gemv_tune that restores the launch table
    on exit."""

    def __init__(self, variant: str | None, balance: bool = True):
        self.variant, self.balance = variant, balance

    def __enter__(self):
        nvfp4_gemv_tune(self.variant, self.balance)
        return self

    def __exit__(self, *exc):
        nvfp4_gemv_tune(None, True)
        return False


def nvfp4_workspace_init(ws, stream=None) -> None:
    _check(lib().nvfp4_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "nvfp4_workspace_init")


def new_workspace(nbytes: int, device="cuda", stream=None):
    """A zero-filled workspace tensor of at least nbytes (16-byte multiple)."""
    import torch

    n = max(16, (int(nbytes) + 15) // 16 * 16)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    nvfp4_workspace_init(ws, stream)
    return ws


def nvfp4_pack_weights(w, ws=None, out: NvFp4Tensor | None = None, stream=None) -> NvFp4Tensor:
    """Pack W fp32 [N][K] (device, contiguous) into NVFP4."""
    import torch

    if w.dim() != 2:
        raise ValueError("w must be [N][K]")
    N, K = int(w.shape[0]), int(w.shape[1])
    _require(w, "w", torch.float32, w.device)
    if out is None:
        out = NvFp4Tensor(torch.empty((N, K // 2), dtype=torch.uint8, device=w.device),
                          torch.empty((N, K // 16), dtype=torch.uint8, device=w.device),
                          torch.empty(1, dtype=torch.float32, device=w.device))
    _require(out.codes, "out.codes", torch.uint8, w.device, (N, K // 2))
    _require(out.scales, "out.scales", torch.uint8, w.device, (N, K // 16))
    _require(out.gscale, "out.gscale", torch.float32, w.device, min_numel=1)
    need = nvfp4_workspace_size(NVFP4_OP_PACK, 0, N, K)
    if ws is None:
        ws = new_workspace(need, w.device, stream)
    _require_ws(ws, need, w.device)
    _check(lib().nvfp4_pack_weights(_ptr(w), N, K, _ptr(out.codes), _ptr(out.scales), _ptr(out.gscale),
                                    _ptr(ws), ws.numel(), _stream(stream)), "nvfp4_pack_weights")
    return out


def nvfp4_quantize_act(x, gscale=None, ws=None, out: NvFp4Tensor | None = None, stream=None,
                       per_token: bool = False) -> NvFp4Tensor:
    """Quantize x bf16 [M][K] (device, contiguous).  ``gscale=None``: dynamic
    global scale (written into out.gscale); else a device fp32 tensor holding
    a static scale (used as out.gscale).  ``per_token``: one global scale per
    row (out.gscale [M]) instead of one for the tensor ([1])."""
    import torch

    if x.dim() != 2:
        raise ValueError("x must be [M][K]")
    M, K = int(x.shape[0]), int(x.shape[1])
    dev = x.device
    _require(x, "x", torch.bfloat16, dev)
    ng = M if per_token else 1
    if gscale is not None:
        _require(gscale, "gscale", torch.float32, dev, min_numel=ng)
    if per_token:
        flags = NVFP4_GS_TOKEN_DYNAMIC if gscale is None else NVFP4_GS_TOKEN_STATIC
    else:
        flags = NVFP4_GS_DYNAMIC if gscale is None else NVFP4_GS_STATIC
    if out is None:
        out = NvFp4Tensor(torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                          torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
                          gscale if gscale is not None else torch.empty(ng, dtype=torch.float32, device=dev))
    _require(out.codes, "out.codes", torch.uint8, dev, (M, K // 2))
    _require(out.scales, "out.scales", torch.uint8, dev, (M, K // 16))
    _require(out.gscale, "out.gscale", torch.float32, dev, min_numel=ng)
    if gscale is not None and out.gscale.data_ptr() != gscale.data_ptr():
        raise ValueError("a static gscale must be out.gscale")
    need = 0 if per_token else nvfp4_workspace_size(NVFP4_OP_QUANT, M, 0, K)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _require_ws(ws, need, dev)
    _check(lib().nvfp4_quantize_act(_ptr(x), M, K, _ptr(out.codes), _ptr(out.scales), _ptr(out.gscale),
                                    flags, _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "nvfp4_quantize_act")
    return out


def nvfp4_quantize_act_rotated(x, rot: int = 16, gscale=None, ws=None, out: NvFp4Tensor | None = None,
                               stream=None) -> NvFp4Tensor:
    """Q+R: rotate each run of ``rot`` elements of every row of x bf16 [M][K]
    by the normalized Walsh-Hadamard matrix, then quantize (dynamic global
    scale, or the static device fp32 ``gscale``, which is then out.gscale)."""
    import torch

    if x.dim() != 2:
        raise ValueError("x must be [M][K]")
    M, K = int(x.shape[0]), int(x.shape[1])
    dev = x.device
    _require(x, "x", torch.bfloat16, dev)
    if gscale is not None:
        _require(gscale, "gscale", torch.float32, dev, min_numel=1)
    flags = NVFP4_GS_DYNAMIC if gscale is None else NVFP4_GS_STATIC
    if out is None:
        out = NvFp4Tensor(torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                          torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
                          gscale if gscale is not None else torch.empty(1, dtype=torch.float32, device=dev))
    _require(out.codes, "out.codes", torch.uint8, dev, (M, K // 2))
    _require(out.scales, "out.scales", torch.uint8, dev, (M, K // 16))
    _require(out.gscale, "out.gscale", torch.float32, dev, min_numel=1)
    if gscale is not None and out.gscale.data_ptr() != gscale.data_ptr():
        raise ValueError("a static gscale must be out.gscale")
    need = nvfp4_workspace_size(NVFP4_OP_QUANT_ROTATED, M, rot, K) if gscale is None else 0
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _require_ws(ws, need, dev)
    _check(lib().nvfp4_quantize_act_rotated(_ptr(x), M, K, int(rot), _ptr(out.codes), _ptr(out.scales),
                                            _ptr(out.gscale), flags, _ptr(ws), 0 if ws is None else ws.numel(),
                                            _stream(stream)),
           "nvfp4_quantize_act_rotated")
    return out


def nvfp4_gemv_variant(M: int, N: int, K: int, lmhead: bool = False) -> str:
    """Kernel variant the library launches for this shape."""
    return lib().nvfp4_gemv_variant(M, N, K, int(bool(lmhead))).decode()


def nvfp4_gemv_variant_names() -> list[str]:
    """Every compiled GEMV kernel variant (names usable in nvfp4_gemv_tune)."""
    out, i = [], 0
    while True:
        n = lib().nvfp4_gemv_variant_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


def variant_tokens(name: str) -> int:
    """Compiled token count of a variant name (``..._m<MT>_...``)."""
    return int(name.split("_m")[1].split("_")[0])


def variant_k_multiple(name: str) -> int:
    """K granularity a variant needs: the streaming kernels (``stream_*``,
    ``fstream_*``, ``wstream_*``) stream whole 512-element chunks (the
    eight-token ``stream8_*`` 256-element ones), the direct-to-LDS kernels
    (``dma_*``, ``staged_*``, ``fmma_*``) and the tiled GEMM (``gemm_*``)
    copy whole 256-element steps, every other kernel 32-element chunks."""
    if name.startswith("stream8_"):
        return 256
    if name.startswith(("stream_", "fstream_", "wstream_")):
        return 512
    return 256 if name.startswith(("dma_", "staged_", "fmma_", "gemm_")) else 32


def nvfp4_reset_state_size(window: int) -> int:
    return int(lib().nvfp4_reset_state_size(window))


def nvfp4_reset_state_init(state, M: int, window: int, stream=None) -> None:
    _check(lib().nvfp4_reset_state_init(_ptr(state), M, window, _stream(stream)), "nvfp4_reset_state_init")


def new_reset_state(M: int, window: int, device="cuda", stream=None):
    import torch

    st = torch.empty(M * nvfp4_reset_state_size(window), dtype=torch.uint8, device=device)
    nvfp4_reset_state_init(st, M, window, stream)
    return st


@dataclass
class Epilogue:
    """Host description of the LM-head epilogue (device tensors inside)."""

    step_start: "object"     # uint8 [M]
    state: "object"          # uint8 [M * state_size]
    entropy: "object"        # fp32 [M]
    temperature: "object"    # fp32 [M]
    tau0: float = 0.6
    t_low: float = 0.4
    t_high: float = 1.0
    t_base: float = 0.6
    window: int = 8
    mode: int = 0            # 0 = ReSET, 1 = BASE (t_base), 2 = fixed threshold tau0

    def as_c(self) -> LmheadEpilogue:
        return LmheadEpilogue(self.tau0, self.t_low, self.t_high, self.t_base, self.window, self.mode,
                              _ptr(self.step_start), _ptr(self.state), _ptr(self.entropy),
                              _ptr(self.temperature))


def _gemv_args(a: NvFp4Tensor, w: NvFp4Tensor, y, epi: Epilogue | None, M: int | None):
    """Check a GEMV's tensors; returns (M, N, K, y, per_token, C epilogue)."""
    import torch

    dev = w.codes.device
    for name, t in (("a.codes", a.codes), ("a.scales", a.scales), ("w.codes", w.codes), ("w.scales", w.scales)):
        _require(t, name, torch.uint8, dev)
        if t.dim() != 2:
            raise ValueError(f"{name} must be 2-D")
    N, K = w.rows, w.K
    if a.K != K:
        raise ValueError(f"activation K {a.K} != weight K {K}")
    M = a.rows if M is None else int(M)
    if not 1 <= M <= a.rows:
        raise ValueError(f"M must be in [1, {a.rows}], got {M}")
    _require(a.scales, "a.scales", torch.uint8, dev, (a.rows, K // 16))
    _require(w.scales, "w.scales", torch.uint8, dev, (N, K // 16))
    _require(w.gscale, "w.gscale", torch.float32, dev, min_numel=1)
    _require(a.gscale, "a.gscale", torch.float32, dev, min_numel=1)
    per_token = a.gscale.numel() > 1
    if per_token and a.gscale.numel() < M:
        raise ValueError(f"per-token a.gscale holds {a.gscale.numel()} scales, {M} needed")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _require(y, "y", torch.float32, dev, (M, N))
    ce = None
    if epi is not None:
        _require(epi.step_start, "epi.step_start", torch.uint8, dev, min_numel=M)
        _require(epi.state, "epi.state", torch.uint8, dev, min_numel=M * nvfp4_reset_state_size(epi.window))
        _require(epi.entropy, "epi.entropy", torch.float32, dev, min_numel=M)
        _require(epi.temperature, "epi.temperature", torch.float32, dev, min_numel=M)
        ce = epi.as_c()
    return M, N, K, y, per_token, ce


def nvfp4_gemv_smallm(a: NvFp4Tensor, w: NvFp4Tensor, y=None, epi: Epilogue | None = None, ws=None,
                      M: int | None = None, stream=None):
    """y [M][N] fp32 = dequant(a) . dequant(w)^T.  ``ws``: a zero-filled
    workspace of at least nvfp4_workspace_size(...) bytes (allocated here
    when needed and not given).  ``M`` (default: a's rows) may use only the
    first rows of ``a``.  An activation with one global scale per row goes
    to the per-token entry point."""
    import torch

    M, N, K, y, per_token, ce = _gemv_args(a, w, y, epi, M)
    dev = w.codes.device
    need = nvfp4_workspace_size(NVFP4_OP_GEMV_LMHEAD if epi is not None else NVFP4_OP_GEMV, M, N, K)
    if need and ws is None:
        ws = new_workspace(need, dev, stream)  # zero-filled: the epilogue's tickets start at zero
    _require_ws(ws, need, dev)
    ws_bytes = 0 if ws is None else ws.numel()
    fn = lib().nvfp4_gemv_smallm_token_scales if per_token else lib().nvfp4_gemv_smallm
    _check(fn(M, N, K, _ptr(a.codes), _ptr(a.scales), _ptr(a.gscale), _ptr(w.codes), _ptr(w.scales),
              _ptr(w.gscale), _ptr(y), None if ce is None else ctypes.byref(ce), _ptr(ws), ws_bytes,
              _stream(stream)), "nvfp4_gemv_smallm")
    return y


def nvfp4_gemv_smallm_noalloc(a: NvFp4Tensor, w: NvFp4Tensor, y=None, epi: Epilogue | None = None,
                              M: int | None = None, stream=None):
    """nvfp4_gemv_smallm with its workspace in the library's static device
    scratch (the entry point for callers that cannot allocate; one global
    activation scale).  ``y`` must be given to allocate nothing here either."""
    M, N, K, y, per_token, ce = _gemv_args(a, w, y, epi, M)
    if per_token:
        raise ValueError("nvfp4_gemv_smallm_noalloc takes one activation global scale")
    _check(lib().nvfp4_gemv_smallm_noalloc(M, N, K, _ptr(a.codes), _ptr(a.scales), _ptr(a.gscale), _ptr(w.codes),
                                           _ptr(w.scales), _ptr(w.gscale), _ptr(y),
                                           None if ce is None else ctypes.byref(ce), _stream(stream)),
           "nvfp4_gemv_smallm_noalloc")
    return y


def nvfp4_sample_top_p(logits, temperature, top_p: float, uniforms, tokens=None, nucleus=None, ws=None,
                       stream=None):
    """One top-p draw per row of ``logits`` [M][N] fp32 at ``temperature``
    [M] fp32 with the caller's ``uniforms`` [M] fp32 in [0, 1).  ``ws``: a
    workspace of nvfp4_workspace_size(NVFP4_OP_SAMPLE, M, N, 0) bytes
    (allocated here when not given; no zero-fill needed).  Returns
    (tokens int32 [M], nucleus sizes int32 [M])."""
    import torch

    M, N = logits.shape
    dev = logits.device
    need = nvfp4_workspace_size(NVFP4_OP_SAMPLE, M, N, 0)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if tokens is None:
        tokens = torch.empty(M, dtype=torch.int32, device=dev)
    if nucleus is None:
        nucleus = torch.empty(M, dtype=torch.int32, device=dev)
    for t, dt in ((logits, torch.float32), (temperature, torch.float32), (uniforms, torch.float32),
                  (tokens, torch.int32), (nucleus, torch.int32)):
        if not t.is_contiguous() or t.dtype != dt or t.device != dev:
            raise ValueError(f"nvfp4_sample_top_p needs contiguous {dt} tensors on {dev}")
    if temperature.numel() != M or uniforms.numel() != M or tokens.numel() != M or nucleus.numel() != M:
        raise ValueError("temperature, uniforms, tokens and nucleus hold one value per row")
    _check(lib().nvfp4_sample_top_p(M, N, _ptr(logits), _ptr(temperature), float(top_p), _ptr(uniforms),
                                    _ptr(tokens), _ptr(nucleus), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)), "nvfp4_sample_top_p")
    return tokens, nucleus
