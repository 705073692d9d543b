"""Benchmark of the NVFP4 small-M decode projection on one MI355X.

Workload: the four Qwen3-32B decode projections (fused QKV 10240x5120,
o_proj 5120x8192, fused gate_up 51200x5120, down_proj 5120x25600) at
M = 1, 2, 4 and 8 active tokens.  One step = for every M and every
projection, quantize the bf16 activation on the GPU (the per-layer "Q" step)
and run the GEMV against the packed NVFP4 weights: 16 quantize launches and
16 GEMV launches.  Inputs are seeded synthetic tensors (workloads/), resident
in HBM before timing starts.  Every projection has enough packed copies
that its launches cycle through at least 576 MB of distinct weights
(2 x (256 MB Infinity Cache + 32 MB L2)), so no GEMV finds its weights in a
cache from an earlier launch.

A step is captured once in a HIP graph (as a decode loop replays it; the
dispatch choices are fixed at capture) and replayed.

Prints one JSON line:
  value        effective GB/s over the step = weight+scale bytes streamed per
               step / step time (quantization included)
  roofline     the GEMV kernel: algorithmic bytes of all GEMV launches of a
               step / their summed average durations (each case: `reps`
               back-to-back launches captured in a graph, HIP events around
               its replay on the launch stream), against the 8 TB/s HBM peak
               and the measured read-stream ceiling: the fastest plain read of
               the same bytes (probe library, best variant and grid per size),
               timed the same way
  cpu_baseline the CPU oracle (quantize + dequantize + fp64 GEMV) on a
               bounded row sample of the same projections, same byte formula,
               with the median time of every (projection, M) case
  extra        the single 4096 x 4096 GEMV and the Qwen3-8B projections at
               M = 1, 2, 4, 8 (per-kernel times, fractions of 8 TB/s and of the
               measured read ceiling), the four projections at M = 16, 32, 64
               and 128 (beyond the metric's M range; per-kernel times only),
               the LM head (N=151936) with the entropy / ReSET epilogue and the
               top-p = 0.95 draw at the epilogue's temperatures, the
               64-layer decode chain captured in one graph, and the
               rotation-fused quantization (Q+R) of the step's activations
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs and effective HBM GB/s per NVFP4 GEMV at M=1/2/4/8; % of HBM peak"
HBM_PEAK_GBS = 8000.0
M_LIST = (1, 2, 4, 8)
M_WIDE = (16, 32, 64, 128)  # beyond the metric's M = 1..8: reported under extra.wide only
CPU_ROWS = 2048

# Measured HBM traffic of the 16 GEMV launches of one step: rocprofv3
# FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a plain
# 512 MiB device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  Valid only for the
# kernel source it was measured on; reported as null once that changes.
GEMV_TRAFFIC = {
    "source": "fp4_decode_gemv_amd/csrc/nvfp4_gemv.hip",
    "sha256": "058ee307d21b18473b3a3fc5a8b7955c46032ccbc7f31afb1129094d710f65d3",
    "bytes_per_step": 1105972704,
}


def measured_traffic():
    import hashlib

    try:
        src = open(os.path.join(ROOT, GEMV_TRAFFIC["source"]), "rb").read()
    except OSError:
        return None
    if hashlib.sha256(src).hexdigest() != GEMV_TRAFFIC["sha256"]:
        return None
    return GEMV_TRAFFIC["bytes_per_step"]


def n_copies(args, c) -> int:
    """Packed copies of a projection: enough to cycle through args.rotate_mb
    of distinct weights, and at least 2."""
    return max(2, math.ceil(args.rotate_mb * 1e6 / weight_bytes(c.N, c.K)))


# dense f16 MFMA peak of MI355X (2.5 PFLOP/s, no sparsity)
MFMA_F16_PEAK_FLOPS = 2.5e15

# VALU issue peak of the chip: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_LANE_OPS_PER_S = 256 * 4 * 16 * 2.4e9


def valu_ops_per_element(variant: str, M: int) -> float:
    """Estimated VALU operations per weight element of a GEMV variant, from
    its decode and dot-product instruction counts: the E2M1 -> f16 decode
    with the block-scale multiply (1 per element), the activation decode of
    the MFMA kernels (shared by the R row tiles, once per 16-token column
    tile), or the f16 dot2 work of the VALU kernels."""
    kind = variant.split("_")[0]
    f = {t[0]: int(t[1:]) for t in variant.split("_")[1:] if t[:1] in "mr" and t[1:].isdigit()}
    mt, r = f.get("m", 8), f.get("r", 1)
    ct = max(1, mt // 16)
    if kind == "direct":
        return 1.1 + 0.6 * M / r
    if kind in ("staged", "valu"):
        return 0.5 + 0.56 * M + (0.5 / r if kind == "staged" else 0.0)
    if kind == "fmma":
        return mt / 8 + 0.2
    if kind == "lmfma":
        return 1 + ct / r
    return 1 + 1 / r  # dma, mfma


def weight_bytes(N: int, K: int) -> int:
    """Algorithmic bytes of one GEMV: codes + E4M3 scales + global scale."""
    return N * K // 2 + N * K // 16 + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate-mb", type=float, default=576.0,
                    help="distinct packed weight bytes (MB) each projection's launches cycle through: at least "
                         "2 x (256 MB Infinity Cache + 32 MB L2), so no launch reads its weights from a cache")
    ap.add_argument("--reps", type=int, default=30, help="timed launches per (projection, M) for per-kernel times")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="rough CPU budget of the oracle baseline")
    ap.add_argument("--no-lmhead", action="store_true", help="skip the LM-head + ReSET epilogue figures")
    ap.add_argument("--no-chain", action="store_true", help="skip the 64-layer hipGraph chain figures")
    ap.add_argument("--no-wide", action="store_true", help="skip the M = 16, 32, 64 and 128 projection figures (extra.wide)")
    ap.add_argument("--no-small", action="store_true", help="skip the 4096 x 4096 and Qwen3-8B projection figures")
    ap.add_argument("--no-probe", action="store_true", help="skip the measured read-stream ceiling")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="at the end, fill and copy a buffer of this many MiB three times: a plain copy of "
                         "known size to calibrate hardware byte counters against")
    ap.add_argument("--proj", default=None,
                    help="comma-separated subset of the projections (qkv,o,gate_up,down) for the step and the "
                         "per-kernel timings, e.g. for a counter profile of a few cases; default: all four")
    ap.add_argument("--m", default=None,
                    help="comma-separated subset of the token counts 1,2,4,8; default: all four")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()
    args.m_list = M_LIST if args.m is None else tuple(int(v) for v in args.m.split(","))
    if not set(args.m_list) <= set(M_LIST):
        ap.error(f"--m takes values out of {M_LIST}")
    args.proj_list = None if args.proj is None else tuple(args.proj.split(","))
    args.subset = args.m is not None or args.proj is not None
    return args


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def setup(args, cases=None, Ms=None):
    """Pack every case's weights on the GPU (enough copies to rotate through
    args.rotate_mb) and make its activations for each M."""
    import torch

    import fp4_decode_gemv_amd as F
    import workloads as W

    dev = torch.device("cuda:0")
    if cases is None:
        cases = [c for c in W.qwen3_32b_cases()
                 if args.proj_list is None or any(c.name in (p, "qwen3_32b_" + p) for p in args.proj_list)]
        if not cases:
            raise SystemExit(f"--proj matches none of {[c.name for c in W.qwen3_32b_cases()]}")
    if Ms is None:
        Ms = args.m_list + (M_WIDE if not args.no_wide else ())
    wq = {}      # name -> list of NvFp4Tensor copies
    samples = {}  # name -> (first CPU_ROWS rows of W, global scale of the whole W)
    for c in cases:
        t0 = time.perf_counter()
        w = W.weights(c.w_seed, c.N, c.K, c.w_outlier_rows)
        samples[c.name] = (w[:CPU_ROWS].copy(), float(np.max(np.abs(w))))
        wt = torch.from_numpy(w).to(dev)
        del w
        base = F.nvfp4_pack_weights(wt)
        del wt
        copies = [base]
        for _ in range(n_copies(args, c) - 1):
            copies.append(F.NvFp4Tensor(base.codes.clone(), base.scales.clone(), base.gscale.clone()))
        wq[c.name] = copies
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        log(args, f"[setup] packed {c.name} {c.N}x{c.K} x{len(copies)} in {time.perf_counter() - t0:.1f}s")
    acts = {}
    for c in cases:
        for M in Ms:
            acts[(c.name, M)] = make_activation(c, M, dev)
    torch.cuda.synchronize()
    return cases, wq, acts, samples


def make_activation(c, M, dev):
    """bf16 input, quantized-activation buffers, workspaces and output of one
    (projection, M) case, resident on the device."""
    import torch

    import fp4_decode_gemv_amd as F
    import workloads as W

    bits = W.case_activations_bf16(c, M)
    x = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16).contiguous()
    aq = F.NvFp4Tensor(torch.empty((M, c.K // 2), dtype=torch.uint8, device=dev),
                       torch.empty((M, c.K // 16), dtype=torch.uint8, device=dev),
                       torch.empty(1, dtype=torch.float32, device=dev))
    need = F.nvfp4_workspace_size(F.NVFP4_OP_QUANT, M, 0, c.K)
    ws = F.new_workspace(need, dev) if need else None
    need = F.nvfp4_workspace_size(F.NVFP4_OP_GEMV, M, c.N, c.K)
    gws = F.new_workspace(need, dev) if need else None
    y = torch.empty((M, c.N), dtype=torch.float32, device=dev)
    return (x, aq, ws, gws, y)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the design notes describe "
              "how the projection would shard). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp4_decode_gemv_amd as F

    F.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    cases, wq, acts, samples = setup(args)
    # one non-default stream (default priority) for capture, replay and events
    stream = torch.cuda.Stream()

    def gemv(c, M, copy):
        x, aq, ws, gws, y = acts[(c.name, M)]
        copies = wq[c.name]
        F.nvfp4_gemv_smallm(aq, copies[copy % len(copies)], y=y, ws=gws, stream=stream)

    def quant(c, M):
        x, aq, ws, gws, y = acts[(c.name, M)]
        F.nvfp4_quantize_act(x, ws=ws, out=aq, stream=stream)

    def step():
        # the four launches of a projection in a step read four different
        # packed copies; between two reads of one copy a whole step (1.1 GB of
        # other weights) goes by, so a replayed step finds nothing in a cache
        for mi, M in enumerate(args.m_list):
            for c in cases:
                quant(c, M)
                gemv(c, M, mi)

    def capture(fn):
        with torch.cuda.stream(stream):
            fn()  # eager run first: nothing is lazily initialised inside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        torch.cuda.synchronize()
        return g

    # ---------------- whole-step throughput (graph replay) ----------------
    g_step = capture(step)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            g_step.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            g_step.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    bytes_per_step = sum(weight_bytes(c.N, c.K) for c in cases) * len(args.m_list)
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    log(args, f"[bench] {ms_per_step * 1e3:.1f} us/step, {value:.0f} GB/s effective (quantization included)")
    del g_step

    # the same step with one activation global scale per token (the
    # quantization's per-token option, which needs no tensor-wide amax; not
    # the metric's per-tensor recipe, so it is reported apart from `value`)
    tok_out = {k: F.nvfp4_quantize_act(v[0], per_token=True) for k, v in acts.items() if k[1] in args.m_list}

    def step_token():
        for mi, M in enumerate(args.m_list):
            for c in cases:
                x, _, _, gws, y = acts[(c.name, M)]
                at = tok_out[(c.name, M)]
                F.nvfp4_quantize_act(x, out=at, stream=stream, per_token=True)
                copies = wq[c.name]
                F.nvfp4_gemv_smallm(at, copies[mi % len(copies)], y=y, ws=gws, stream=stream)

    g_tok = capture(step_token)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            g_tok.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            g_tok.replay()
    torch.cuda.synchronize()
    tok_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    token_scales = {"ms_per_step": round(tok_ms, 4),
                    "gbs": round(bytes_per_step / (tok_ms * 1e-3) / 1e9, 1)}
    log(args, f"[bench] per-token scales: {tok_ms * 1e3:.1f} us/step, {token_scales['gbs']:.0f} GB/s effective")
    del g_tok

    # the same step launched eagerly from Python, for reference (host-bound)
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    te = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(10):
            step()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - te) * 1e3 / 10
    log(args, f"[bench] eager Python launches: {eager_ms * 1e3:.1f} us/step")

    # ---------------- per-kernel durations ----------------
    # `reps` launches of one case back to back, captured in a graph and
    # timed by HIP events on the launch stream around its replay: the
    # average is the kernel's duration as a decode step runs it (it agrees
    # with rocprofv3's per-dispatch durations); host launch overhead is not
    # in it.
    detail = time_cases(args, stream, cases, wq, acts, args.m_list, with_valu=True)
    gemv_bytes = sum(d["weight_bytes"] for d in detail)
    gemv_us = sum(d["gemv_us"] for d in detail)
    achieved = gemv_bytes / (gemv_us * 1e-6) / 1e9

    extra = {"eager_python_launch_ms_per_step": round(eager_ms, 4), "token_scales": token_scales}
    # the rotation-fused quantization (Q+R) of the same activations, the
    # pages' comparison point for the Q step
    extra["q_plus_r"] = time_q_plus_r(args, stream, cases, acts, detail)
    if not args.no_wide:
        # 16, 32, 64 and 128 tokens (1, 2, 4 or 8 16-token MFMA column tiles): the
        # same per-kernel timing, outside the step and the roofline figures
        extra["wide"] = time_cases(args, stream, cases, wq, acts, M_WIDE)
    copies_rotated = {c.name: len(wq[c.name]) for c in cases}
    del wq, acts
    torch.cuda.empty_cache()

    # ---------------- measured read-stream ceiling ----------------
    import workloads as W

    small_cases = [W.single_case()] + W.qwen3_8b_cases()
    sizes = {weight_bytes(c.N, c.K) for c in cases + small_cases}
    if not args.no_lmhead:
        sizes.add(weight_bytes(W.lm_head_case().N, W.lm_head_case().K))
    ceiling = read_ceiling(args, stream, sizes) if not args.no_probe else {}
    for d in detail:
        _attach_ceiling(d, ceiling)
    probe_us = sum(ceiling[d["weight_bytes"]]["us"] for d in detail) if ceiling else None
    extra["read_ceiling"] = {str(k): v for k, v in sorted(ceiling.items())}

    # ---------------- the 4096 x 4096 GEMV and the Qwen3-8B projections ----------------
    if not args.no_small:
        sc, swq, sacts, _ = setup(args, small_cases, M_LIST)
        small = time_cases(args, stream, sc, swq, sacts, M_LIST)
        for d in small:
            _attach_ceiling(d, ceiling)
        extra["single_4096"] = [d for d in small if d["proj"] == "square_4096"]
        extra["qwen3_8b"] = [d for d in small if d["proj"] != "square_4096"]
        del swq, sacts
        torch.cuda.empty_cache()

    if not args.no_lmhead:
        extra["lm_head"] = bench_lm_head(args, stream)
    if not args.no_chain:
        extra["chain"] = bench_chain(args, stream)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            src.fill_(1)
            dst.copy_(src)
        torch.cuda.synchronize()
        log(args, f"[copy-probe] filled and copied {n} bytes x3")
        del src, dst

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args, cases, samples)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-32B decode projections, NVFP4 W4A4: qkv 10240x5120, o 5120x8192, "
                        "gate_up 51200x5120, down 5120x25600; M in {1,2,4,8}; one step = activation "
                        "quantization + GEMV for each (projection, M)",
            "global_batch": list(args.m_list),
            "weight_bytes_per_step": bytes_per_step,
            "weight_copies_rotated": copies_rotated,
            "parallelism": "single-gpu",
            **({"subset": {"proj": list(args.proj_list or ()), "m": list(args.m_list)}} if args.subset else {}),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "measured_ceiling": None if probe_us is None else round(gemv_bytes / (probe_us * 1e-6) / 1e9, 1),
            "frac_of_measured_ceiling": None if probe_us is None else round(probe_us / gemv_us, 4),
            "measured_ceiling_note": "the fastest plain read of each case's weight bytes on this GPU (probe library: "
                                     "best of its register-ring and LDS-ring variants over 256..2048 workgroups, timed "
                                     "like the GEMVs, rotated past the caches), summed over the 16 cases",
            "traffic": measured_traffic(),
            "traffic_unit": "HBM bytes read + written by the 16 GEMV launches of one step (rocprofv3 "
                            "FETCH_SIZE / WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes": gemv_bytes,
            "kernel": "gemv kernels, all 16 (projection, M) cases of a step: summed algorithmic bytes / summed "
                      "average launch durations (per case: `reps` back-to-back launches captured in a HIP graph, "
                      "HIP events around its replays on the launch stream)",
        },
        "cpu_baseline": cpu,
        "detail": detail,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def time_cases(args, stream, cases, wq, acts, Ms, with_valu=False):
    """Per-kernel duration of the GEMV and of the activation quantization of
    every (case, M): `reps` back-to-back launches captured in one graph (each
    GEMV on the next packed copy of its weights), 7 timed replays."""
    import fp4_decode_gemv_amd as F

    def gemv(c, M, copy):
        x, aq, ws, gws, y = acts[(c.name, M)]
        copies = wq[c.name]
        F.nvfp4_gemv_smallm(aq, copies[copy % len(copies)], y=y, ws=gws, stream=stream)

    def quant(c, M):
        x, aq, ws, gws, y = acts[(c.name, M)]
        F.nvfp4_quantize_act(x, ws=ws, out=aq, stream=stream)

    def b2b(fn):
        return _graph_us(fn, args.reps, stream, replays=7)  # >= 200 timed dispatches per case

    rows = []
    for c in cases:
        for M in Ms:
            gus = b2b(lambda i: gemv(c, M, i))
            qus = b2b(lambda i: quant(c, M))
            wb = weight_bytes(c.N, c.K)
            v = F.nvfp4_gemv_variant(M, c.N, c.K)
            d = {"proj": c.name, "M": M, "N": c.N, "K": c.K, "weight_bytes": wb, "variant": v,
                 "gemv_us": round(gus, 3), "gemv_gbs": round(wb / (gus * 1e-6) / 1e9, 1),
                 "gemv_hbm_frac": round(wb / (gus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "quant_us": round(qus, 3),
                 # the useful multiply-adds (M tokens, not the padded tiles) against the dense f16 MFMA peak
                 "tflops": round(2.0 * M * c.N * c.K / (gus * 1e-6) / 1e12, 2),
                 "mfma_f16_frac": round(2.0 * M * c.N * c.K / (gus * 1e-6) / MFMA_F16_PEAK_FLOPS, 4)}
            if with_valu:
                # estimated VALU issue utilisation (the secondary ceiling at larger M)
                d["valu_util_est"] = round(valu_ops_per_element(v, M) * c.N * c.K / (gus * 1e-6) / VALU_LANE_OPS_PER_S, 3)
            rows.append(d)
            log(args, f"[kern] {c.name:18s} M={M:<3d} gemv {gus:8.2f} us {wb / (gus * 1e-6) / 1e9:7.0f} GB/s "
                      f"({wb / (gus * 1e-6) / 1e9 / HBM_PEAK_GBS * 100:4.1f}% of 8 TB/s)  quant {qus:6.2f} us  {v}")
    return rows


def time_q_plus_r(args, stream, cases, acts, detail):
    """Per-launch time of the rotation-fused quantization (block Walsh-Hadamard
    rotation of 16 and of 128 elements, then the NVFP4 recipe) next to the
    plain quantization of the same (projection, M) cases."""
    import fp4_decode_gemv_amd as F

    q_us = {(d["proj"], d["M"]): d["quant_us"] for d in detail}
    rows = []
    for c in cases:
        for M in args.m_list:
            x, aq, ws, gws, y = acts[(c.name, M)]
            row = {"proj": c.name, "M": M, "K": c.K, "quant_us": q_us[(c.name, M)]}
            for R in (16, 128):
                need = F.nvfp4_workspace_size(F.NVFP4_OP_QUANT_ROTATED, M, R, c.K)
                rws = F.new_workspace(need, x.device) if need else None
                us = _graph_us(lambda i: F.nvfp4_quantize_act_rotated(x, R, ws=rws, out=aq, stream=stream),
                               args.reps, stream, replays=7)
                row[f"quant_rot{R}_us"] = round(us, 3)
            row["rot16_over_quant"] = round(row["quant_rot16_us"] / row["quant_us"], 3)
            rows.append(row)
            log(args, f"[q+r] {c.name:18s} M={M:<3d} Q {row['quant_us']:.2f} us, Q+R(16) {row['quant_rot16_us']:.2f} us, "
                      f"Q+R(128) {row['quant_rot128_us']:.2f} us")
    return rows


def read_ceiling(args, stream, sizes):
    """For each byte count: the fastest plain read of that many bytes (the
    probe library's register-ring and LDS-ring variants over 256..2048
    workgroups), each launch on the next copy of a rotation past the caches,
    timed like the GEMVs.  (A wider search, every variant over 128..4096
    workgroups, found the same best times within 2%.)"""
    import torch

    from fp4_decode_gemv_amd import probe as P

    names = P.read_variants()
    cand = [names.index(n) for n in ("vgpr_u2_1", "vgpr_u4_1", "vgpr_u8_1", "vgpr_u16_1", "lds_d4") if n in names]
    pool_bytes = 1400 << 20
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda:0")
    pool.fill_(1)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    out = {}
    for nb in sorted(sizes):
        b16 = nb // 16 * 16  # the probe reads whole 16-byte units (the 4-byte global scale left out)
        stride = (b16 + 4095) // 4096 * 4096
        ncop = max(1, pool_bytes // stride)
        reps = min(ncop, max(20, math.ceil(600e6 / b16)))
        best = None
        for vi in cand:
            for grid in (256, 512, 768, 1024, 1536, 2048):
                us = _graph_us(lambda i: P.read(vi, pool[(i % ncop) * stride:], b16, grid, sink, stream), reps, stream)
                if best is None or us < best[0]:
                    best = (us, names[vi], grid)
        out[nb] = {"us": round(best[0], 3), "gbs": round(nb / (best[0] * 1e-6) / 1e9, 1),
                   "hbm_frac": round(nb / (best[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "variant": best[1], "grid": best[2]}
        log(args, f"[ceiling] {nb / 1e6:8.2f} MB: {best[0]:7.2f} us {out[nb]['gbs']:7.0f} GB/s ({best[1]}, grid {best[2]})")
    del pool
    torch.cuda.empty_cache()
    return out


def _attach_ceiling(d, ceiling):
    c = ceiling.get(d["weight_bytes"])
    if c:
        d["read_ceiling_us"] = c["us"]
        d["frac_of_read_ceiling"] = round(c["us"] / d["gemv_us"], 4)


def _replay_us(g, reps, stream, replays=5):
    """Average microseconds per launch of a graph holding `reps` launches:
    one warm replay, then the mean over `replays` replays (HIP events on the
    replay stream)."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * replays)


def _graph_us(fn, reps, stream, replays=5):
    """Capture `reps` calls of fn(i) in a graph on `stream` and time it."""
    import torch

    with torch.cuda.stream(stream):
        fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fn(i)
    torch.cuda.synchronize()
    us = _replay_us(g, reps, stream, replays)
    del g
    return us


def bench_lm_head(args, stream):
    """LM head N=151936 K=5120 at M = 1 and 8: quantization + GEMV with the
    fused entropy / ReSET epilogue, the plain GEMV for comparison, and the
    top-p = 0.95 draw at the epilogue's temperatures (alone and as the tail
    of the decode step), and on flat synthetic rows."""
    import torch

    import fp4_decode_gemv_amd as F
    import workloads as W

    dev = torch.device("cuda:0")
    case = W.lm_head_case()
    w = W.chain_weights_gpu(case, dev)
    base = F.nvfp4_pack_weights(w)
    del w
    copies = [base, F.NvFp4Tensor(base.codes.clone(), base.scales.clone(), base.gscale.clone())]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    wb = weight_bytes(case.N, case.K)
    out = []
    for M in (1, 8):
        x = torch.from_numpy(W.activations_bf16(case.x_seed, case.K, M).view(np.int16)).to(dev).view(torch.bfloat16)
        aq = F.nvfp4_quantize_act(x)
        qn = F.nvfp4_workspace_size(F.NVFP4_OP_QUANT, M, 0, case.K)
        qws = F.new_workspace(qn, dev) if qn else None
        y = torch.empty((M, case.N), device=dev)
        st = F.new_reset_state(M, 8, dev)
        epi = F.Epilogue(step_start=torch.zeros(M, dtype=torch.uint8, device=dev), state=st,
                         entropy=torch.empty(M, device=dev), temperature=torch.empty(M, device=dev), window=8)
        ews = F.new_workspace(F.nvfp4_workspace_size(F.NVFP4_OP_GEMV_LMHEAD, M, case.N, case.K), dev)
        gn = F.nvfp4_workspace_size(F.NVFP4_OP_GEMV, M, case.N, case.K)
        gws = F.new_workspace(gn, dev) if gn else None
        uni = torch.from_numpy(W.sampler_uniforms(3500, 1, M)[0]).to(dev)
        tok = torch.empty(M, dtype=torch.int32, device=dev)
        nuc = torch.empty(M, dtype=torch.int32, device=dev)
        sws = torch.empty(F.nvfp4_workspace_size(F.NVFP4_OP_SAMPLE, M, case.N, 0), dtype=torch.uint8, device=dev)

        def sample(i):
            F.nvfp4_sample_top_p(y, epi.temperature, 0.95, uni, tokens=tok, nucleus=nuc, ws=sws, stream=stream)

        def decode_tail(i):
            F.nvfp4_quantize_act(x, ws=qws, out=aq, stream=stream)
            F.nvfp4_gemv_smallm(aq, copies[i % 2], y=y, epi=epi, ws=ews, stream=stream)
            sample(i)

        def with_epi(i):
            F.nvfp4_quantize_act(x, ws=qws, out=aq, stream=stream)
            F.nvfp4_gemv_smallm(aq, copies[i % 2], y=y, epi=epi, ws=ews, stream=stream)

        def epi_only(i):
            F.nvfp4_gemv_smallm(aq, copies[i % 2], y=y, epi=epi, ws=ews, stream=stream)

        def plain(i):
            F.nvfp4_gemv_smallm(aq, copies[i % 2], y=y, ws=gws, stream=stream)

        t_all = _graph_us(with_epi, args.reps, stream)
        t_epi = _graph_us(epi_only, args.reps, stream)
        t_plain = _graph_us(plain, args.reps, stream)
        t_tail = _graph_us(decode_tail, args.reps, stream)
        t_samp = _graph_us(sample, args.reps, stream)  # logits and temperatures of the last step
        # a flat row (N(0, 1) logits at T = 1: the nucleus holds most of the
        # vocabulary), which takes the histogram path of the draw
        gen = torch.Generator(device=dev)
        gen.manual_seed(3600 + M)
        z_flat = torch.randn((M, case.N), device=dev, generator=gen)
        t_one = torch.ones(M, device=dev)

        def sample_flat(i):
            F.nvfp4_sample_top_p(z_flat, t_one, 0.95, uni, tokens=tok, nucleus=nuc, ws=sws, stream=stream)

        t_flat = _graph_us(sample_flat, args.reps, stream)
        del z_flat
        out.append({"M": M, "N": case.N, "K": case.K, "weight_bytes": wb,
                    "variant": F.nvfp4_gemv_variant(M, case.N, case.K, True),
                    "quant_gemv_epilogue_us": round(t_all, 2), "gemv_epilogue_us": round(t_epi, 2),
                    "gemv_plain_us": round(t_plain, 2), "gemv_epilogue_gbs": round(wb / t_epi / 1e3, 1),
                    "epilogue_overhead_us": round(t_epi - t_plain, 2),
                    "sample_top_p_us": round(t_samp, 2), "sample_top_p_flat_rows_us": round(t_flat, 2),
                    "quant_gemv_epilogue_sample_us": round(t_tail, 2)})
        log(args, f"[lmhead] M={M} quant+gemv+epilogue {t_all:.2f} us, gemv+epilogue {t_epi:.2f} us "
                  f"({wb / t_epi / 1e3:.0f} GB/s), plain gemv {t_plain:.2f} us, top-p draw {t_samp:.2f} us "
                  f"(flat rows {t_flat:.2f} us), "
                  f"whole tail {t_tail:.2f} us")
    del copies, base
    torch.cuda.empty_cache()
    return out


def bench_chain(args, stream):
    """64 Qwen3-32B layers x 4 projections (17.55 GB of packed weights)
    captured in one hipGraph; microseconds per decode step at M = 1 and 8:
    with the dynamic per-tensor, dynamic per-token or static activation
    quantization before each GEMV, and GEMV-only."""
    import torch

    import fp4_decode_gemv_amd as F
    import workloads as W

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    ws = {}
    for l in range(W.CHAIN_LAYERS):
        for p in range(4):
            c = W.chain_case(l, p)
            wt = W.chain_weights_gpu(c, dev)
            ws[(l, p)] = F.nvfp4_pack_weights(wt)
            del wt
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    total = sum(weight_bytes(W.chain_case(0, p).N, W.chain_case(0, p).K) for p in range(4)) * W.CHAIN_LAYERS
    log(args, f"[chain] packed {W.CHAIN_LAYERS}x4 projections ({total / 1e9:.2f} GB) in {time.perf_counter() - t0:.1f}s")
    out = []
    for M in (1, 8):
        io = {}
        for l in range(W.CHAIN_LAYERS):
            for p in range(4):
                c = W.chain_case(l, p)
                x = torch.from_numpy(W.chain_activations_bf16(l, p, M).view(np.int16)).to(dev).view(torch.bfloat16)
                aq = F.nvfp4_quantize_act(x)
                at = F.nvfp4_quantize_act(x, per_token=True)
                # a calibrated (static) global scale: the dynamic one of this input, taken once
                ast = F.nvfp4_quantize_act(x, gscale=aq.gscale.clone())
                qn = F.nvfp4_workspace_size(F.NVFP4_OP_QUANT, M, 0, c.K)
                gn = F.nvfp4_workspace_size(F.NVFP4_OP_GEMV, M, c.N, c.K)
                io[(l, p)] = (x, aq, at, ast, F.new_workspace(qn, dev) if qn else None,
                              F.new_workspace(gn, dev) if gn else None, torch.empty((M, c.N), device=dev))
        res = {"M": M, "weight_bytes": total}
        # per-tensor dynamic quantization + GEMV, per-token dynamic quantization
        # + GEMV, static (calibrated) per-tensor scale + GEMV, GEMV alone
        for key in ("quant_gemv", "token_quant_gemv", "static_quant_gemv", "gemv_only"):
            def step(_i):
                for l in range(W.CHAIN_LAYERS):
                    for p in range(4):
                        x, aq, at, ast, qws, gws, y = io[(l, p)]
                        a = aq
                        if key == "quant_gemv":
                            F.nvfp4_quantize_act(x, ws=qws, out=aq, stream=stream)
                        elif key == "token_quant_gemv":
                            F.nvfp4_quantize_act(x, out=at, stream=stream, per_token=True)
                            a = at
                        elif key == "static_quant_gemv":
                            F.nvfp4_quantize_act(x, gscale=ast.gscale, out=ast, stream=stream)
                            a = ast
                        F.nvfp4_gemv_smallm(a, ws[(l, p)], y=y, ws=gws, stream=stream)
            us = _graph_us(step, 1, stream)
            res[key + "_us_per_step"] = round(us, 1)
            res[key + "_gbs"] = round(total / us / 1e3, 1)
        out.append(res)
        log(args, f"[chain] M={M} {res['quant_gemv_us_per_step']:.1f} us/step with quantization "
                  f"({res['quant_gemv_gbs']:.0f} GB/s), {res['token_quant_gemv_us_per_step']:.1f} us with "
                  f"per-token scales, {res['static_quant_gemv_us_per_step']:.1f} us with a static scale, "
                  f"{res['gemv_only_us_per_step']:.1f} us GEMV only "
                  f"({res['gemv_only_gbs']:.0f} GB/s)")
        del io
    del ws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(args, cases, samples):
    """Time the oracle on the host: activation quantization plus dequantize +
    fp64 GEMV over a row sample of each projection (M = 1..8 as in a step),
    with the median time of every (projection, M) case."""
    from oracle import nvfp4_oracle as O
    import workloads as W

    rows = CPU_ROWS
    t_start = time.perf_counter()
    # pack the sampled rows with the oracle (weight packing is offline, not timed)
    packed = {}
    for c in cases:
        w, amax = samples[c.name]
        packed[c.name] = O.quantize_nvfp4(w, O.global_scale(amax))
    xs = {(c.name, M): W.case_activations_bf16(c, M) for c in cases for M in args.m_list}
    runs, per_case = [], {(c.name, M): [] for c in cases for M in args.m_list}
    for _ in range(7):
        t0 = time.perf_counter()
        for M in args.m_list:
            for c in cases:
                tc = time.perf_counter()
                aq = O.quantize_act_bf16(xs[(c.name, M)])
                O.gemv_ref(aq, packed[c.name])
                per_case[(c.name, M)].append(time.perf_counter() - tc)
        runs.append(time.perf_counter() - t0)
        if len(runs) >= 3 and time.perf_counter() - t_start > args.cpu_seconds:
            break
    t = float(np.median(runs))
    sample_bytes = sum(weight_bytes(rows, c.K) for c in cases) * len(args.m_list)
    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    cases_out = []
    for c in cases:
        for M in args.m_list:
            tc = float(np.median(per_case[(c.name, M)]))
            cases_out.append({"proj": c.name, "M": M, "rows": rows, "us": round(tc * 1e6, 1),
                              "gbs": round(weight_bytes(rows, c.K) / tc / 1e9, 4)})
    return {
        "value": round(sample_bytes / t / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {rows} weight rows of each of the 4 projections x M in {{1,2,4,8}} "
                  f"(activation quantization + dequantize + fp64 GEMV), median of {len(runs)} runs, "
                  f"{t * 1e3:.0f} ms per sampled step; host {os.cpu_count()} logical CPUs",
        "cases": cases_out,
    }


if __name__ == "__main__":
    main()
