"""GPU parity of the top-p sampler against the oracle.

The kernel computes probabilities as float32 exponentials summed in 2^-40
fixed point; the oracle sorts and sums in float64.  Their normalised
cumulative masses differ by at most DELTA: the exponent (z - z_max) log2(e)/T
carries three float32 roundings (relative 3 * 2^-24 of an exponent a), so an
exponential is off by at most ln2 * 3 * 2^-24 * a + 2 ulp; weighted by the
probabilities, a averages at most log2(N) bits (17.3 for the LM head), which
bounds the relative error of any partial sum by 2.3e-6; fixed-point
truncation adds N * 2^-40 relative to the row maximum (1.4e-7); the ratio
of two such sums doubles the bound.  A GPU draw is accepted when some
nucleus size and some draw point within DELTA of the oracle's select it,
and must equal the oracle's draw when no cut point lies within DELTA."""

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
import workloads as W
from gpu_util import bf16_dev, f32_dev
from oracle import sampler_oracle as S

pytestmark = pytest.mark.gpu

DELTA = 5e-6


def _check_row(z, T, top_p, u, tok, nuc):
    """Validity of one GPU draw; returns True when it had to be exact."""
    order, c = S.sorted_cumulative(z, T)
    N = c.size
    rank = np.empty(N, dtype=np.int64)
    rank[order] = np.arange(N)
    n_lo = min(int(np.searchsorted(c, top_p - DELTA, side="left")) + 1, N)
    n_hi = min(int(np.searchsorted(c, top_p + DELTA, side="left")) + 1, N)
    assert n_lo <= nuc <= n_hi, ("nucleus", nuc, n_lo, n_hi)
    k = int(rank[tok])
    assert k < nuc, ("token outside its nucleus", k, nuc)
    r = u * c[nuc - 1]
    lo = c[k - 1] if k > 0 else 0.0
    assert lo <= r + DELTA and c[k] >= r - DELTA, ("draw", k, lo, c[k], r)
    ref_tok, ref_n = S.sample_top_p(z, T, top_p, u)
    kr = int(rank[ref_tok])
    lor = c[kr - 1] if kr > 0 else 0.0
    # every admissible nucleus puts the draw point well inside the oracle
    # token's interval: the token is unique
    clear = lor < u * c[n_lo - 1] - 2 * DELTA and c[kr] > u * c[n_hi - 1] + 2 * DELTA
    if clear:
        assert tok == ref_tok, ("unambiguous draw differs", tok, ref_tok)
    if n_lo == n_hi:
        assert nuc == ref_n
    return clear


def _run(z, T, top_p, u):
    tok, nuc = F.nvfp4_sample_top_p(f32_dev(z), f32_dev(T), top_p, f32_dev(u))
    torch.cuda.synchronize()
    return tok.cpu().numpy(), nuc.cpu().numpy()


def _check(z, T, top_p, u):
    tok, nuc = _run(z, T, top_p, u)
    exact = 0
    for m in range(z.shape[0]):
        exact += _check_row(z[m], float(T[m]), top_p, float(u[m]), int(tok[m]), int(nuc[m]))
    return tok, nuc, exact


@pytest.mark.parametrize("N", [1, 2, 3, 5, 100, 1000, 4099, 65536, 151936])
@pytest.mark.parametrize("top_p", [0.95, 0.5, 1.0, 1e-6])
def test_random_logits(N, top_p):
    print(f"[sampler] N={N} top_p={top_p}", flush=True)
    rng = np.random.default_rng(N * 7 + int(top_p * 1000))
    M = 8
    z = (rng.standard_normal((M, N)) * rng.uniform(0.2, 4.0, (M, 1))).astype(np.float32)
    T = rng.choice([0.1, 0.4, 0.6, 1.0, 1.7], M).astype(np.float32)
    u = rng.random(M).astype(np.float32)
    tok, nuc, exact = _check(z, T, top_p, u)
    if N <= 1000:
        assert exact >= M // 2, exact   # most draws are far from every cut point
    if top_p == 1e-6:
        assert np.all(tok == np.argmax(z, axis=1)) and np.all(nuc == 1)


def _run_flags(z, T, top_p, u):
    """Draws plus the per-row flag of the listed path (1: the token was
    drawn from launch 1's short lists), read from the sampler's workspace,
    whose layout ends with that [M] int32 array padded to 256 bytes.  The
    workspace starts out filled with 0xFF bytes: it needs no zero-fill."""
    M, N = z.shape
    dev = torch.device("cuda:0")
    need = F.nvfp4_workspace_size(F.NVFP4_OP_SAMPLE, M, N, 0)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    tok, nuc = F.nvfp4_sample_top_p(f32_dev(z), f32_dev(T), top_p, f32_dev(u), ws=ws)
    torch.cuda.synchronize()
    off = need - (M * 4 + 255) // 256 * 256
    flags = ws[off:off + 4 * M].view(torch.int32).cpu().numpy()
    return tok.cpu().numpy(), nuc.cpu().numpy(), flags


def _peaked_rows(N, seed):
    """Eight rows over an N(0, 2) bulk: k spikes in [35, 60] spread evenly
    over the row, k = 1, 3 (three equal maxima), 8, 40, 120, 250, then 300
    spikes in [59, 60], and bulk only.  The first launch lists a chunk's
    elements within 20 log2(e)-units (13.9 T) of its maximum, at most 32:
    on the 4096-element chunks of the long rows a spike chunk holds at most 7
    spikes, so every spike within 13.9 T of the row maximum is listed and the
    rest of the row is below 1e-5 of its mass; rows 0 to 5 are drawn by the
    listed path for any top_p < 1.  Row 6 lists more elements than the
    path ranks (256) and row 7's chunks all overflow: both take the
    histogram path.  On short rows (one or two chunks) the spikes of rows 4
    and 5 overflow their chunk as well."""
    rng = np.random.default_rng(seed)
    z = (2.0 * rng.standard_normal((8, N))).astype(np.float32)
    for m, k in enumerate((1, 3, 8, 40, 120, 250, 300, 0)):
        if k == 0:
            continue
        idx = np.unique(np.linspace(0, N - 1, min(k, N)).astype(np.int64))
        lo = 59.0 if m == 6 else 35.0
        z[m, idx] = rng.uniform(lo, 60.0, idx.size).astype(np.float32)
        if k == 3:
            z[m, idx] = np.float32(50.0)
    T = np.array([0.6, 1.0, 1.7, 0.6, 1.0, 1.7, 1.0, 1.0], dtype=np.float32)
    return z, T


@pytest.mark.parametrize("N", [151936, 151937, 4099, 1000])
@pytest.mark.parametrize("top_p", [0.95, 0.5, 1e-6, 1.0])
def test_peaked_rows_one_launch_path(N, top_p):
    """Rows whose nucleus lies among a few high logits are drawn from the
    first launch's short lists (flag read back from the workspace), mixed in
    one call with rows that need the histogram path; all against the oracle.  N = 151937
    takes the scalar loads, 4099 a 3-element last chunk, 1000 one chunk."""
    print(f"[sampler peaked] N={N} top_p={top_p}", flush=True)
    z, T = _peaked_rows(N, 40 + N % 97)
    u = np.random.default_rng(N + 3).random(8).astype(np.float32)
    tok, nuc, flags = _run_flags(z, T, top_p, u)
    for m in range(8):
        _check_row(z[m], float(T[m]), top_p, float(u[m]), int(tok[m]), int(nuc[m]))
    assert set(np.unique(flags)) <= {0, 1}, flags
    if top_p < 1.0:
        if N > 100000:
            assert np.all(flags[:6] == 1), flags
        else:
            assert np.all(flags[:4] == 1) and np.all(flags[4:6] == 0), flags
    assert flags[6] == 0 and flags[7] == 0, flags
    if top_p == 1e-6:
        assert np.all(tok == np.argmax(z, axis=1)) and np.all(nuc == 1)
    # the three equal maxima are drawn in index order
    if top_p < 1.0:
        top3 = np.flatnonzero(z[1] == np.float32(50.0))
        assert tok[1] in top3


def test_peaked_rows_past_the_listed_path_length():
    """Rows of more than 256 chunks of 4096 (N > 1M) always take the
    histogram path, peaked or not."""
    N = 1_100_000
    print(f"[sampler long] N={N}", flush=True)
    z, T = _peaked_rows(N, 41)
    z, T = z[[0, 3]], T[[0, 3]]
    u = np.array([0.3, 0.8], dtype=np.float32)
    tok, nuc, flags = _run_flags(z, T, 0.95, u)
    assert np.all(flags == 0), flags
    for m in range(2):
        _check_row(z[m], float(T[m]), 0.95, float(u[m]), int(tok[m]), int(nuc[m]))


def test_equal_logits_take_index_order():
    """All logits equal: every element lands in one bucket and shares one key,
    so the cut points come from the tie walk; the closed form is exact."""
    N, M = 5000, 6
    z = np.full((M, N), 0.75, dtype=np.float32)
    T = np.full(M, 0.6, dtype=np.float32)
    u = np.array([0.0, 0.1234, 0.5, 0.77, 0.99, 0.31], dtype=np.float32)
    for top_p in (0.95, 0.5, 1.0):
        tok, nuc = _run(z, T, top_p, u)
        n = int(np.ceil(np.float64(np.float32(top_p)) * N))
        assert np.all(nuc == n), (top_p, nuc, n)
        assert np.array_equal(tok, np.floor(u.astype(np.float64) * n).astype(np.int64)), (top_p, tok)


def test_near_flat_logits_refine_by_key_bits():
    """Logits within 1e-5 of each other: one level-0 bucket holds the row, the
    key-bit refinement has to narrow it down."""
    rng = np.random.default_rng(9)
    M, N = 8, 20000
    z = (1.0 + 1e-5 * rng.standard_normal((M, N))).astype(np.float32)
    T = np.full(M, 1.0, dtype=np.float32)
    u = rng.random(M).astype(np.float32)
    _check(z, T, 0.95, u)
    _check(z, T, 0.3, u)


def test_large_bucket_inside_the_collected_list():
    """600 near-equal logits (one bucket) hold most of the mass: the list of
    collected elements does not overflow, but the cut's bucket is larger than
    the directly ranked set, so the selection narrows it in LDS by key bits
    before ranking."""
    rng = np.random.default_rng(16)
    M, N = 8, 20000
    z = np.full((M, N), -30.0, dtype=np.float32)
    for m in range(M):
        idx = rng.choice(N, 603, replace=False)
        z[m, idx[:600]] = (0.005 * rng.random(600)).astype(np.float32)
        z[m, idx[600:]] = np.array([1.0, 2.0, 3.0], dtype=np.float32)
    T = np.full(M, 1.0, dtype=np.float32)
    u = rng.random(M).astype(np.float32)
    for top_p in (0.95, 0.5):
        tok, nuc, exact = _check(z, T, top_p, u)
        assert exact >= M // 2, exact


@pytest.mark.parametrize("layout", ["one_chunk", "spread"])
def test_collected_list_overflow_takes_the_passes(layout):
    """3000 near-equal logits carrying most of the mass, either inside one
    4096-element chunk (that chunk's workgroup gathers more than it can hold
    and marks the list incomplete) or spread over the row with 5000 of them
    (the row's list of 4096 overflows): the selection falls back to the
    passes over the row."""
    rng = np.random.default_rng(21 if layout == "one_chunk" else 22)
    M, N = 4, 60000
    z = np.full((M, N), -40.0, dtype=np.float32)
    for m in range(M):
        if layout == "one_chunk":
            idx = 8192 + rng.choice(4096, 3000, replace=False)
        else:
            idx = rng.choice(N, 5000, replace=False)
        z[m, idx] = (0.004 * rng.random(idx.size)).astype(np.float32)
    T = np.full(M, 1.0, dtype=np.float32)
    u = rng.random(M).astype(np.float32)
    for top_p in (0.95, 0.3):
        _check(z, T, top_p, u)


def test_flat_rows_on_the_full_vocabulary():
    """Near-uniform rows of 151936 logits (the nucleus holds most of the
    vocabulary; the cut buckets hold hundreds of elements each)."""
    rng = np.random.default_rng(23)
    M, N = 4, 151936
    z = (rng.standard_normal((M, N)) * np.array([[0.3], [1.0], [2.0], [3.0]])).astype(np.float32)
    T = np.array([1.0, 1.0, 0.8, 0.6], dtype=np.float32)
    u = rng.random(M).astype(np.float32)
    _check(z, T, 0.95, u)


def test_few_distinct_values_with_many_ties():
    rng = np.random.default_rng(10)
    M, N = 8, 12000
    z = (rng.integers(0, 6, (M, N)) * 0.25).astype(np.float32)
    z[:, ::7] = -0.0
    z[:, 1::7] = 0.0
    T = np.full(M, 0.5, dtype=np.float32)
    u = rng.random(M).astype(np.float32)
    for top_p in (0.95, 0.6, 0.2):
        _check(z, T, top_p, u)


def test_sharp_rows_and_extreme_temperatures():
    rng = np.random.default_rng(12)
    M, N = 8, 30000
    z = (rng.standard_normal((M, N)) * 64.0).astype(np.float32)      # H near 0
    T = np.array([1e-3, 0.05, 0.4, 1.0, 10.0, 100.0, 1e4, 0.6], dtype=np.float32)
    u = rng.random(M).astype(np.float32)
    _check(z, T, 0.95, u)


def test_invalid_temperature_and_clamped_uniforms():
    rng = np.random.default_rng(13)
    M, N = 6, 777
    z = rng.standard_normal((M, N)).astype(np.float32)
    T = np.array([0.0, -1.0, np.nan, np.inf, 1.0, 1.0], dtype=np.float32)
    u = np.array([0.5, 0.5, 0.5, 0.5, 1.5, -0.25], dtype=np.float32)
    tok, nuc = _run(z, T, 0.9, u)
    assert list(tok[:4]) == [-1] * 4 and list(nuc[:4]) == [0] * 4
    last = S.nucleus_order(z[4])[nuc[4] - 1]      # u >= 1 draws the nucleus's last token
    assert tok[4] == last
    assert tok[5] == int(np.argmax(z[5]))         # u < 0 draws the top token


@pytest.mark.parametrize("peaked", [False, True])
def test_repeatable_and_graph_replays_match_eager(peaked):
    """Repeated calls and graph replays on one workspace (never cleared
    between calls): identical draws."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(14)
    M, N = 8, 151936
    if peaked:
        zh, Th = _peaked_rows(N, 17)
        z, T = f32_dev(zh), f32_dev(Th)
    else:
        z = f32_dev((rng.standard_normal((M, N)) * 3.0).astype(np.float32))
        T = f32_dev(np.full(M, 0.6, dtype=np.float32))
    u = f32_dev(rng.random(M).astype(np.float32))
    ws = torch.full((F.nvfp4_workspace_size(F.NVFP4_OP_SAMPLE, M, N, 0),), 0xFF, dtype=torch.uint8, device=dev)
    tok, nuc = F.nvfp4_sample_top_p(z, T, 0.95, u, ws=ws)
    torch.cuda.synchronize()
    ref = (tok.cpu().numpy().copy(), nuc.cpu().numpy().copy())
    for _ in range(3):
        t2, n2 = F.nvfp4_sample_top_p(z, T, 0.95, u, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(t2.cpu().numpy(), ref[0]) and np.array_equal(n2.cpu().numpy(), ref[1])
    s = torch.cuda.Stream()
    tg = torch.empty(M, dtype=torch.int32, device=dev)
    ng = torch.empty(M, dtype=torch.int32, device=dev)
    with torch.cuda.stream(s):
        F.nvfp4_sample_top_p(z, T, 0.95, u, tokens=tg, nucleus=ng, ws=ws, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        F.nvfp4_sample_top_p(z, T, 0.95, u, tokens=tg, nucleus=ng, ws=ws, stream=s)
    for _ in range(4):
        tg.fill_(-7)
        ng.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tg.cpu().numpy(), ref[0]) and np.array_equal(ng.cpu().numpy(), ref[1])


def test_lm_head_decode_step():
    """Quantize, LM-head GEMV with the ReSET epilogue, then sample at the
    epilogue's temperatures: the full decode tail on the LM-head shape."""
    dev = torch.device("cuda:0")
    case = W.lm_head_case()
    print(f"[sampler lmhead] N={case.N} K={case.K}", flush=True)
    w = W.weights(case.w_seed, case.N, case.K, case.w_outlier_rows)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    del w
    torch.cuda.empty_cache()
    rng = np.random.default_rng(15)
    for M in (1, 8):
        xs = W.lm_head_positions_bf16(case.x_seed, 2, M, case.K)
        st = F.new_reset_state(M, 8, dev)
        ent, tmp = torch.empty(M, device=dev), torch.empty(M, device=dev)
        ws = F.new_workspace(F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, M, case.N, case.K), dev)
        flags = torch.ones(M, dtype=torch.uint8, device=dev)
        for t in range(2):
            aq = F.nvfp4_quantize_act(bf16_dev(xs[t]))
            y = F.nvfp4_gemv_smallm(aq, wq, epi=F.Epilogue(flags, st, ent, tmp, window=8), ws=ws)
            u = rng.random(M).astype(np.float32)
            tok, nuc = F.nvfp4_sample_top_p(y, tmp, 0.95, f32_dev(u))
            torch.cuda.synchronize()
            z, T = y.cpu().numpy(), tmp.cpu().numpy()
            tok, nuc = tok.cpu().numpy(), nuc.cpu().numpy()
            for m in range(M):
                _check_row(z[m], float(T[m]), 0.95, float(u[m]), int(tok[m]), int(nuc[m]))
