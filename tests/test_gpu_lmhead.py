"""GPU parity of the fused LM-head epilogue: entropy within 1e-4 nats of the
fp64 entropy of the GPU's own logits, and ReSET temperatures equal to the
oracle's wherever the decision is not within the rounding band of a tie."""

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
import workloads as W
from oracle import nvfp4_oracle as O
from oracle import reset_oracle as R
from gpu_util import assert_gemv_close, bf16_dev, f32_dev, oracle_rows_ref

pytestmark = pytest.mark.gpu

BAND = 1e-9   # rounding band for decisions fed with the GPU's own entropies


def _decisions_agree(tr: R.ResetTrace, T_gpu: np.ndarray, p: R.ResetParams, band: float):
    """Compare T where neither comparison of the oracle is within `band` of a tie."""
    tie = (np.abs(tr.Hstep - tr.Hbar) < band) | (np.abs(tr.H - tr.tau) < band)
    ok = (T_gpu.astype(np.float64) == np.float32(tr.T).astype(np.float64)) | tie
    return ok, int(tie.sum())


def _run_sequence(wq, xbits_pos, flags, p: R.ResetParams, M, scale_exp=None, keep=None):
    """Decode `positions` steps; returns the logits of the kept positions
    (all by default, else {t: logits} for t in `keep`), H [P][M], T [P][M]
    and, for every position, the fp64 entropy of the GPU's own logits."""
    dev = torch.device("cuda:0")
    P = xbits_pos.shape[0]
    st = F.new_reset_state(M, p.window, dev)
    ent = torch.empty(M, device=dev)
    tmp = torch.empty(M, device=dev)
    ws = F.new_workspace(F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, M, wq.rows, wq.K), dev)
    Hs, Ts, Hrefs = [], [], []
    logits = [] if keep is None else {}
    for t in range(P):
        xb = xbits_pos[t]
        aq = F.nvfp4_quantize_act(bf16_dev(xb))
        if scale_exp is not None:
            aq.gscale.mul_(float(2.0 ** scale_exp[t]))
        f = torch.from_numpy(np.ascontiguousarray(flags[t])).to(dev)
        epi = F.Epilogue(step_start=f, state=st, entropy=ent, temperature=tmp, tau0=p.tau0, t_low=p.t_low,
                         t_high=p.t_high, t_base=p.t_base, window=p.window, mode=p.mode)
        y = F.nvfp4_gemv_smallm(aq, wq, epi=epi, ws=ws)
        Hs.append(ent.cpu().numpy().copy())
        Ts.append(tmp.cpu().numpy().copy())
        yh = y.cpu().numpy()
        Hrefs.append(R.entropy_rows(yh.astype(np.float64)))
        if keep is None:
            logits.append(yh)
        elif t in keep:
            logits[t] = yh
    return logits, np.array(Hs), np.array(Ts), np.array(Hrefs)


@pytest.mark.parametrize("mode,M,N,K", [(0, 4, 3000, 512), (1, 4, 3000, 512), (2, 4, 3000, 512), (0, 1, 2500, 1024),
                                         (0, 8, 2000, 8192), (0, 2, 4099, 256), (0, 16, 3000, 512), (2, 13, 2500, 1024),
                                         (0, 32, 3000, 512), (1, 23, 2500, 1024), (0, 64, 3000, 512),
                                         (2, 41, 2500, 1024), (0, 128, 3000, 512), (1, 77, 2500, 1024),
                                         (0, 12, 70000, 256), (0, 6, 70000, 256)])
def test_small_vocab_sequence(mode, M, N, K):
    P = 60
    w = W.small_random_weights(41, N, K, scale=0.2)
    rng = np.random.default_rng(42)
    xs = np.stack([W.small_random_bf16(100 + t, M, K) for t in range(P)])
    u = rng.integers(0, 7, P)                 # activation scale 2^u: exact, spans H in ~[0, ln N]
    flags = W.step_flags(43, P, M, p=0.15)
    p = R.ResetParams(tau0=0.6, t_low=0.4, t_high=1.0, t_base=0.6, window=4, mode=mode)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    logits, H, T, Href = _run_sequence(wq, xs, flags, p, M, scale_exp=u)
    for t in range(P):
        assert np.all(np.abs(H[t] - Href[t]) <= 1e-4), (t, H[t], Href[t])
    assert H.min() < 0.6 < H.max(), "sequence must exercise both sides of tau0"
    ties = 0
    for m in range(M):
        tr = R.reset_sequence(H[:, m].astype(np.float32).astype(np.float64), flags[:, m], p)
        ok, nt = _decisions_agree(tr, T[:, m], p, BAND)
        ties += nt
        assert ok.all(), (m, np.nonzero(~ok))
        if mode == 1:
            assert np.all(T[:, m] == np.float32(0.6))
        if mode == 2:
            Hm = H[:, m].astype(np.float64)
            clear = np.abs(Hm - p.tau0) >= BAND
            assert np.all(T[clear, m] == np.where(Hm[clear] < p.tau0, np.float32(p.t_low), np.float32(p.t_high)))
    # logits of the last step against the oracle
    wr = O.quantize_nvfp4(w)
    ar = O.quantize_act_bf16(xs[-1])
    ar = (ar[0], ar[1], np.float32(ar[2] * np.float32(2.0 ** u[-1])))
    y_ref, ref_abs = O.gemv_ref(ar, wr)
    assert_gemv_close(logits[-1], y_ref, ref_abs, what="lm logits")


def test_one_token_tile_sizes_agree():
    """One token on an LM-head-sized vocabulary: the launch table's 16-row
    tiles (4375 partials) and the 8-row tiles of another direct form (8750,
    forced)
    give the same entropies within rounding, each within 1e-4 nats of the
    fp64 entropy of its own logits, and ReSET decisions that match the
    oracle."""
    M, N, K, P = 1, 70000, 256, 24
    w = W.small_random_weights(61, N, K, scale=0.2)
    xs = np.stack([W.small_random_bf16(300 + t, M, K) for t in range(P)])
    u = np.random.default_rng(62).integers(0, 7, P)
    flags = W.step_flags(63, P, M, p=0.2)
    p = R.ResetParams(window=4)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    assert F.nvfp4_gemv_variant(M, N, K, True) == "direct_m1_g32_r2_w4_p1_nt"
    _, H1, T1, Href1 = _run_sequence(wq, xs, flags, p, M, scale_exp=u)
    with F.forced_variant("direct_m1_g32_r1_w4_p1_nt"):
        assert F.nvfp4_gemv_variant(M, N, K, True) == "direct_m1_g32_r1_w4_p1_nt"
        _, H2, T2, Href2 = _run_sequence(wq, xs, flags, p, M, scale_exp=u)
    assert np.all(np.abs(H1 - Href1) <= 1e-4) and np.all(np.abs(H2 - Href2) <= 1e-4)
    assert np.all(np.abs(H1 - H2) <= 1e-4)
    assert H1.min() < 0.6 < H1.max()
    for H, T in ((H1, T1), (H2, T2)):
        tr = R.reset_sequence(H[:, 0].astype(np.float32).astype(np.float64), flags[:, 0], p)
        ok, _ = _decisions_agree(tr, T[:, 0], p, BAND)
        assert ok.all()


def test_chunked_runs_carry_state():
    """One run of 40 positions equals two runs of 20 with the state kept."""
    M, N, K = 2, 2000, 256
    w = W.small_random_weights(51, N, K, scale=0.3)
    xs = np.stack([W.small_random_bf16(200 + t, M, K) for t in range(40)])
    flags = W.step_flags(52, 40, M, p=0.2)
    p = R.ResetParams(window=3)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    _, H1, T1, _ = _run_sequence(wq, xs, flags, p, M)
    # same thing, state re-initialised only once, in two halves
    dev = torch.device("cuda:0")
    st = F.new_reset_state(M, p.window, dev)
    ent, tmp = torch.empty(M, device=dev), torch.empty(M, device=dev)
    ws = F.new_workspace(F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, M, N, K), dev)
    T2 = []
    for half in (range(0, 20), range(20, 40)):
        for t in half:
            aq = F.nvfp4_quantize_act(bf16_dev(xs[t]))
            f = torch.from_numpy(np.ascontiguousarray(flags[t])).to(dev)
            F.nvfp4_gemv_smallm(aq, wq, epi=F.Epilogue(f, st, ent, tmp, window=p.window), ws=ws)
            T2.append(tmp.cpu().numpy().copy())
    assert np.array_equal(np.array(T2), T1)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("M", [1, 8])
def test_full_lm_head_sequence(M):
    """The LM-head workload end to end: 512 positions of M sequences with
    fresh activations (exponents 2^u spreading the entropies over every
    branch of the rule), seeded step flags, the full 151936-row head.
    Entropies within 1e-4 nats of the fp64 entropy of the GPU's logits at
    every position and, at two positions, of the oracle's own logits over
    the whole vocabulary; temperatures equal to the oracle's ReSET rule
    wherever it is not within rounding of a tie; sampled logits of those two
    positions against the oracle."""
    case = W.lm_head_case()
    P = 512
    print(f"[lmhead] N={case.N} K={case.K} M={M} positions={P}", flush=True)
    w = W.weights(case.w_seed, case.N, case.K, case.w_outlier_rows)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    torch.cuda.empty_cache()
    xs = W.lm_head_positions_bf16(case.x_seed, P, M, case.K)
    flags = W.step_flags(3300, P, M)
    u = W.pow2_exponents(3400, P)
    p = R.ResetParams(tau0=0.6, t_low=0.4, t_high=1.0, t_base=0.6, window=8)
    checked = (0, P - 1)
    logits, H, T, Href = _run_sequence(wq, xs, flags, p, M, scale_exp=u, keep=checked)
    for t in range(P):
        assert np.all(np.abs(H[t] - Href[t]) <= 1e-4), (t, H[t], Href[t])
    for m in range(M):
        tr = R.reset_sequence(H[:, m].astype(np.float32).astype(np.float64), flags[:, m], p)
        ok, _ = _decisions_agree(tr, T[:, m], p, BAND)
        assert ok.all(), (m, np.nonzero(~ok))
    print(f"[lmhead] M={M}: {P} positions checked; oracle logits of positions {checked}", flush=True)
    s_g = O.global_scale(np.max(np.abs(w)))
    ars = []
    for t in checked:
        ar = O.quantize_act_bf16(xs[t])
        ars.append((ar[0], ar[1], np.float32(ar[2] * np.float32(2.0 ** u[t]))))
    for t, (y_ref, ref_abs) in zip(checked, oracle_rows_ref(w, s_g, ars)):
        assert_gemv_close(logits[t], y_ref, ref_abs, what=f"lm head t={t}")
        assert np.all(np.abs(H[t] - R.entropy_rows(y_ref)) <= 1e-4), (t, H[t], R.entropy_rows(y_ref))


@pytest.mark.parametrize("M", [1, 8])
def test_epilogue_graph_replays_match_eager(M):
    """The LM-head call (GEMV, partials, multi-workgroup merge with its
    self-resetting counters) captured in a HIP graph and replayed several
    times, with eager work in between, gives the eager entropies every time;
    the ReSET state advances once per replay exactly as eager calls do."""
    dev = torch.device("cuda:0")
    N, K = 20000, 1024
    print(f"[lmhead graph] M={M} N={N} K={K}", flush=True)
    w = W.small_random_weights(77, N, K, scale=0.2)
    wq = F.nvfp4_pack_weights(f32_dev(w))
    aq = F.nvfp4_quantize_act(bf16_dev(W.small_random_bf16(78, M, K)))
    ws = F.new_workspace(F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, M, N, K), dev)
    flags = torch.zeros(M, dtype=torch.uint8, device=dev)
    ent, tmp = torch.empty(M, device=dev), torch.empty(M, device=dev)
    y = torch.empty((M, N), device=dev)
    s = torch.cuda.Stream()

    def call(st):
        epi = F.Epilogue(step_start=flags, state=st, entropy=ent, temperature=tmp, window=4)
        F.nvfp4_gemv_smallm(aq, wq, y=y, epi=epi, ws=ws, stream=torch.cuda.current_stream())

    # eager reference: four calls on a fresh state
    st_e = F.new_reset_state(M, 4, dev)
    ref_H, ref_T = [], []
    for _ in range(4):
        call(st_e)
        torch.cuda.synchronize()
        ref_H.append(ent.cpu().numpy().copy())
        ref_T.append(tmp.cpu().numpy().copy())
    # graph: capture one call on a second state, replay it four times
    st_g = F.new_reset_state(M, 4, dev)
    st_w = F.new_reset_state(M, 4, dev)
    with torch.cuda.stream(s):
        call(st_w)  # warm-up outside the capture, on a scratch state
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(st_g)
    torch.cuda.synchronize()
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(ent.cpu().numpy(), ref_H[r]), (r, ent.cpu().numpy(), ref_H[r])
        assert np.array_equal(tmp.cpu().numpy(), ref_T[r]), (r, tmp.cpu().numpy(), ref_T[r])
        y.zero_()  # eager work between replays
        torch.cuda.synchronize()


def test_epilogue_workspace_allocated_by_the_binding_starts_at_zero():
    """Without a caller workspace the binding allocates one; its ticket
    counters must start at zero even where the allocator hands back memory
    that held other data (a freed block of the same size filled with 0xFF
    is reused by the caching allocator)."""
    dev = torch.device("cuda:0")
    M, N, K = 4, 5000, 512
    w = W.small_random_weights(91, N, K, scale=0.2)
    xb = W.small_random_bf16(92, M, K)
    wq, aq = F.nvfp4_pack_weights(f32_dev(w)), F.nvfp4_quantize_act(bf16_dev(xb))
    need = F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, M, N, K)
    for _ in range(2):
        junk = torch.full((max(16, (need + 15) // 16 * 16),), 0xFF, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        del junk
        ent = torch.full((M,), float("nan"), device=dev)
        tmp = torch.full((M,), float("nan"), device=dev)
        epi = F.Epilogue(step_start=torch.ones(M, dtype=torch.uint8, device=dev), state=F.new_reset_state(M, 8, dev),
                         entropy=ent, temperature=tmp, window=8)
        y = F.nvfp4_gemv_smallm(aq, wq, epi=epi)
        torch.cuda.synchronize()
        H = ent.cpu().numpy()
        assert np.all(np.isfinite(H)) and np.all(np.isfinite(tmp.cpu().numpy())), (H, tmp)
        assert np.all(np.abs(H - R.entropy_rows(y.cpu().numpy().astype(np.float64))) <= 1e-4)

