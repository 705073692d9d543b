"""Seeded synthetic inputs for the NVFP4 small-M decode projection.

This module only draws random numbers and rounds them to the input dtypes.
It holds none of the method's arithmetic (no quantization, no GEMV, no
entropy), so both the CPU oracle and the HIP path can take their inputs from
it without sharing any of the computation.

Shapes are the Qwen3 projection shapes the ReSET project page lists in its
"Kernel-level decode latency for M=1 GEMV" table, with q/k/v and gate/up
fused into one projection each, plus the Qwen3 LM head (vocabulary 151936,
hidden 5120).

Recipe (stated once, used everywhere):
  * RNG: numpy PCG64 via ``numpy.random.default_rng(seed)``; one generator per
    tensor; ``standard_normal(dtype=float32)``.
  * Weights: ``W = float32(0.02) * N(0,1)`` of shape [N][K].  For the
    "outlier rows" variant, ``floor(0.001*N)`` rows drawn afterwards from the
    same generator with ``choice(N, count, replace=False)`` are multiplied by 8.
  * Activations: ``x = N(0,1)`` of shape [8][K]; ``floor(0.01*K)`` channels
    (columns shared by all rows) drawn afterwards from the same generator are
    multiplied by 20; then rounded to bfloat16 (round-to-nearest-even).
    Smaller M takes the first M rows, so all M share a prefix.
  * SwiGLU activations (input of a down projection): ``x = bf16(silu(g) * u)``
    with g, u ~ N(0,1) float32 from two generators, computed in float32, no
    extra outliers.
  * ReSET step flags: ``rng.random((positions, 8)) < 0.02``, position 0 forced
    to 1.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------
# Shapes (N, K) of one decode projection y[M][N] = A[M][K] . W[N][K]^T
# ---------------------------------------------------------------------------

SINGLE_4096 = {"square": (4096, 4096)}

QWEN3_8B = {
    "qkv": (6144, 4096),        # 32 q heads + 2*4 kv heads, head dim 128
    "o": (4096, 4096),
    "gate_up": (24576, 4096),   # gate and up fused (2 * 12288)
    "down": (4096, 12288),
}

QWEN3_32B = {
    "qkv": (10240, 5120),       # 64 q heads + 2*8 kv heads, head dim 128
    "o": (5120, 8192),
    "gate_up": (51200, 5120),   # gate and up fused (2 * 25600)
    "down": (5120, 25600),
}

LM_HEAD = (151936, 5120)

M_VALUES = (1, 2, 4, 8)

PROJ_ORDER = ("qkv", "o", "gate_up", "down")


@dataclass(frozen=True)
class ProjectionCase:
    """One projection workload: shape, seeds and distribution switches."""

    name: str
    N: int
    K: int
    w_seed: int
    x_seed: int                 # activation seed (g seed for SwiGLU inputs)
    u_seed: int | None = None   # u seed for SwiGLU inputs, else None
    w_outlier_rows: bool = False

    @property
    def swiglu(self) -> bool:
        return self.u_seed is not None


def single_case() -> ProjectionCase:
    N, K = SINGLE_4096["square"]
    return ProjectionCase("square_4096", N, K, 100, 101)


def qwen3_8b_cases() -> list[ProjectionCase]:
    c = []
    for i, p in enumerate(PROJ_ORDER):
        N, K = QWEN3_8B[p]
        if p == "down":
            c.append(ProjectionCase(f"qwen3_8b_{p}", N, K, 1100 + i, 1213, u_seed=1223))
        else:
            c.append(ProjectionCase(f"qwen3_8b_{p}", N, K, 1100 + i, 1200 + i))
    return c


def qwen3_32b_cases() -> list[ProjectionCase]:
    c = []
    for i, p in enumerate(PROJ_ORDER):
        N, K = QWEN3_32B[p]
        c.append(ProjectionCase(f"qwen3_32b_{p}", N, K, 2100 + i, 2200 + i, w_outlier_rows=True))
    return c


def lm_head_case() -> ProjectionCase:
    N, K = LM_HEAD
    return ProjectionCase("qwen3_32b_lm_head", N, K, 3100, 3200, w_outlier_rows=True)


CHAIN_LAYERS = 64
CHAIN_CHECKED_LAYERS = (0, 31, 63)


def chain_case(layer: int, proj_index: int) -> ProjectionCase:
    """Projection ``proj_index`` of layer ``layer`` of the 64-layer chain."""
    p = PROJ_ORDER[proj_index]
    N, K = QWEN3_32B[p]
    return ProjectionCase(
        f"chain_l{layer}_{p}", N, K,
        4_000_000 + 10 * layer + proj_index,
        4_100_000 + 10 * layer + proj_index,
        w_outlier_rows=True,
    )


# ---------------------------------------------------------------------------
# bf16 rounding (input dtype conversion, round-to-nearest-even)
# ---------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (RNE) and return the uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------

def weights(seed: int, N: int, K: int, outlier_rows: bool = False) -> np.ndarray:
    """W fp32 [N][K] = 0.02 * N(0,1); optionally floor(0.001 N) rows * 8."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(0.02)
    if outlier_rows:
        cnt = math.floor(0.001 * N)
        if cnt > 0:
            rows = rng.choice(N, cnt, replace=False)
            w[rows] *= np.float32(8.0)
    return w


def weight_rows(seed: int, N: int, K: int, outlier_rows: bool, rows: np.ndarray) -> np.ndarray:
    """Rows ``rows`` of ``weights(seed, N, K, outlier_rows)``, drawn without
    materialising the whole matrix (the generator is advanced row by row)."""
    rng = np.random.default_rng(seed)
    want = np.asarray(rows, dtype=np.int64)
    order = np.argsort(want)
    out = np.empty((len(want), K), dtype=np.float32)
    chunk = max(1, (64 << 20) // (4 * K))
    pos = 0
    j = 0
    while pos < N and j < len(want):
        n = min(chunk, N - pos)
        block = rng.standard_normal((n, K), dtype=np.float32)
        while j < len(want) and want[order[j]] < pos + n:
            out[order[j]] = block[want[order[j]] - pos]
            j += 1
        pos += n
    # advance past the remaining rows so the outlier draw sees the same state
    while pos < N:
        n = min(chunk, N - pos)
        rng.standard_normal((n, K), dtype=np.float32)
        pos += n
    out *= np.float32(0.02)
    if outlier_rows:
        cnt = math.floor(0.001 * N)
        if cnt > 0:
            orows = set(int(r) for r in rng.choice(N, cnt, replace=False))
            for i, r in enumerate(want):
                if int(r) in orows:
                    out[i] *= np.float32(8.0)
    return out


def outlier_rows_of(seed: int, N: int, K: int) -> np.ndarray:
    """The row indices the outlier-row variant scales by 8 (for test coverage)."""
    rng = np.random.default_rng(seed)
    chunk = max(1, (64 << 20) // (4 * K))
    pos = 0
    while pos < N:
        n = min(chunk, N - pos)
        rng.standard_normal((n, K), dtype=np.float32)
        pos += n
    cnt = math.floor(0.001 * N)
    return np.sort(rng.choice(N, cnt, replace=False)) if cnt else np.zeros(0, np.int64)


def activations_f32(seed: int, K: int, rows: int = 8, outliers: bool = True) -> np.ndarray:
    """Pre-rounding activation x fp32 [rows][K] = N(0,1), 1% of channels * 20."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K), dtype=np.float32)
    if outliers:
        cnt = math.floor(0.01 * K)
        if cnt > 0:
            ch = rng.choice(K, cnt, replace=False)
            x[:, ch] *= np.float32(20.0)
    return x


def activations_bf16(seed: int, K: int, M: int, outliers: bool = True) -> np.ndarray:
    """Activation bf16 bits [M][K] (first M rows of an [8][K] draw)."""
    x = activations_f32(seed, K, max(8, M), outliers)
    return to_bf16_bits(x[:M])


def swiglu_activations_bf16(g_seed: int, u_seed: int, K: int, M: int) -> np.ndarray:
    """bf16 bits [M][K] of silu(g)*u, g,u ~ N(0,1) float32 [8][K]."""
    g = np.random.default_rng(g_seed).standard_normal((max(8, M), K), dtype=np.float32)
    u = np.random.default_rng(u_seed).standard_normal((max(8, M), K), dtype=np.float32)
    one = np.float32(1.0)
    silu = g / (one + np.exp(-g))
    x = (silu * u).astype(np.float32)
    return to_bf16_bits(x[:M])


def case_activations_bf16(case: ProjectionCase, M: int) -> np.ndarray:
    if case.swiglu:
        return swiglu_activations_bf16(case.x_seed, case.u_seed, case.K, M)
    return activations_bf16(case.x_seed, case.K, M)


def lm_head_positions_bf16(seed: int, positions: int, M: int, K: int) -> np.ndarray:
    """Per-position activations bf16 bits [positions][M][K] (outlier channels
    drawn once per position from the same generator after its values)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((positions, 8, K), dtype=np.float32)
    cnt = math.floor(0.01 * K)
    for p in range(positions):
        ch = rng.choice(K, cnt, replace=False)
        x[p][:, ch] *= np.float32(20.0)
    return to_bf16_bits(x[:, :M, :])


def step_flags(seed: int, positions: int, seqs: int = 8, p: float = 0.02) -> np.ndarray:
    """uint8 [positions][seqs]: 1 where a new reasoning step starts (drawn
    for max(8, seqs) sequences, so the first 8 never depend on seqs)."""
    rng = np.random.default_rng(seed)
    f = (rng.random((positions, max(8, seqs))) < p).astype(np.uint8)[:, :seqs]
    f[0, :] = 1
    return f


def sampler_uniforms(seed: int, positions: int, seqs: int = 8) -> np.ndarray:
    """float32 [positions][seqs] in [0, 1): the caller's random numbers for
    the top-p draws (the sampler itself draws none)."""
    rng = np.random.default_rng(seed)
    return rng.random((positions, max(8, seqs)), dtype=np.float32)[:, :seqs].copy()


def pow2_exponents(seed: int, positions: int, hi: int = 6) -> np.ndarray:
    """Integers u ~ U{0..hi} per position (activations scaled by 2**u)."""
    return np.random.default_rng(seed).integers(0, hi + 1, positions)


def small_random_bf16(seed: int, M: int, K: int, scale: float = 1.0) -> np.ndarray:
    """Small ad-hoc activation (no outliers) for parity cases that are not one
    of the named workloads."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(scale)
    return to_bf16_bits(x)


def small_random_weights(seed: int, N: int, K: int, scale: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, K), dtype=np.float32) * np.float32(scale)


def chain_weights_gpu(case: ProjectionCase, device):
    """Weights of an unchecked chain layer, drawn on the GPU with torch's
    seeded generator (same distribution as ``weights``: 0.02 * N(0,1), then
    floor(0.001 N) rows * 8).  Checked layers use ``weights`` instead, so the
    CPU oracle can regenerate them."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(case.w_seed)
    w = torch.randn((case.N, case.K), generator=g, device=device, dtype=torch.float32)
    w.mul_(0.02)
    if case.w_outlier_rows:
        cnt = math.floor(0.001 * case.N)
        if cnt:
            rows = torch.randperm(case.N, generator=g, device=device)[:cnt]
            w[rows] *= 8.0
    return w


def chain_activations_bf16(layer: int, proj_index: int, M: int) -> np.ndarray:
    c = chain_case(layer, proj_index)
    return activations_bf16(c.x_seed, c.K, M)
