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
    the directly ranked set, so the cut takes the passes over the row."""
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


def test_repeatable_and_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(14)
    M, N = 8, 151936
    z = f32_dev((rng.standard_normal((M, N)) * 3.0).astype(np.float32))
    T = f32_dev(np.full(M, 0.6, dtype=np.float32))
    u = f32_dev(rng.random(M).astype(np.float32))
    tok, nuc = F.nvfp4_sample_top_p(z, T, 0.95, u)
    torch.cuda.synchronize()
    ref = (tok.cpu().numpy().copy(), nuc.cpu().numpy().copy())
    for _ in range(3):
        t2, n2 = F.nvfp4_sample_top_p(z, T, 0.95, u)
        torch.cuda.synchronize()
        assert np.array_equal(t2.cpu().numpy(), ref[0]) and np.array_equal(n2.cpu().numpy(), ref[1])
    s = torch.cuda.Stream()
    tg = torch.empty(M, dtype=torch.int32, device=dev)
    ng = torch.empty(M, dtype=torch.int32, device=dev)
    with torch.cuda.stream(s):
        F.nvfp4_sample_top_p(z, T, 0.95, u, tokens=tg, nucleus=ng, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        F.nvfp4_sample_top_p(z, T, 0.95, u, tokens=tg, nucleus=ng, stream=s)
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
