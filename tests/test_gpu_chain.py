"""The 64-layer Qwen3-32B decode-step chain (4 projections per layer, each
activation quantization + GEMV) captured in one hipGraph: every replay equals
the eager run bit for bit, and layers 0, 31 and 63 match the oracle."""

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
import workloads as W
from oracle import nvfp4_oracle as O
from gpu_util import assert_gemv_close, bf16_dev, f32_dev

pytestmark = pytest.mark.gpu


class Chain:
    def __init__(self, Ms, layers=W.CHAIN_LAYERS):
        dev = torch.device("cuda:0")
        self.Ms = Ms
        self.layers = layers
        self.w = {}
        self.checked_w = {}
        for l in range(layers):
            for p in range(4):
                c = W.chain_case(l, p)
                if l in W.CHAIN_CHECKED_LAYERS:
                    wh = W.weights(c.w_seed, c.N, c.K, c.w_outlier_rows)
                    rng = np.random.default_rng(l * 4 + p)
                    rows = np.unique(np.concatenate([[0, c.N - 1], rng.choice(c.N, 24, replace=False)]))
                    self.checked_w[(l, p)] = (rows, O.quantize_nvfp4(wh[rows], O.global_scale(np.max(np.abs(wh)))))
                    wt = f32_dev(wh)
                    del wh
                else:
                    wt = W.chain_weights_gpu(c, dev)
                self.w[(l, p)] = F.nvfp4_pack_weights(wt)
                del wt
            torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.io = {}
        for M in Ms:
            for l in range(layers):
                for p in range(4):
                    c = W.chain_case(l, p)
                    xb = W.chain_activations_bf16(l, p, M)
                    x = bf16_dev(xb)
                    aq = F.NvFp4Tensor(torch.empty((M, c.K // 2), dtype=torch.uint8, device=dev),
                                       torch.empty((M, c.K // 16), dtype=torch.uint8, device=dev),
                                       torch.empty(1, dtype=torch.float32, device=dev))
                    qn = F.nvfp4_workspace_size(F.NVFP4_OP_QUANT, M, 0, c.K)
                    gn = F.nvfp4_workspace_size(F.NVFP4_OP_GEMV, M, c.N, c.K)
                    self.io[(M, l, p)] = dict(xb=xb, x=x, aq=aq, y=torch.empty((M, c.N), device=dev),
                                              qws=F.new_workspace(qn, dev) if qn else None,
                                              gws=F.new_workspace(gn, dev) if gn else None)
        torch.cuda.synchronize()

    def step(self, M, quantize=True):
        for l in range(self.layers):
            for p in range(4):
                io = self.io[(M, l, p)]
                if quantize:
                    F.nvfp4_quantize_act(io["x"], ws=io["qws"], out=io["aq"])
                F.nvfp4_gemv_smallm(io["aq"], self.w[(l, p)], y=io["y"], ws=io["gws"])

    def capture(self, M, quantize=True):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step(M, quantize)          # warm-up outside the graph
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.step(M, quantize)
        torch.cuda.synchronize()
        return g

    def outputs(self, M):
        torch.cuda.synchronize()
        return {k[1:]: v["y"].cpu().numpy().copy() for k, v in self.io.items() if k[0] == M}


@pytest.fixture(scope="module")
def chain():
    print("[chain] building 64 layers x 4 projections", flush=True)
    return Chain((1, 8))


@pytest.mark.parametrize("M", [1, 8])
def test_chain_graph_replays_match_eager_and_oracle(chain, M):
    print(f"[chain] M={M}", flush=True)
    chain.step(M)
    eager = chain.outputs(M)
    g = chain.capture(M)
    for rep in range(3):
        for io in (chain.io[(M, l, p)] for l in range(chain.layers) for p in range(4)):
            io["y"].fill_(float("nan"))        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = chain.outputs(M)
        for k in eager:
            assert np.array_equal(got[k], eager[k]), (rep, k)
    for (l, p), (rows, wr) in chain.checked_w.items():
        io = chain.io[(M, l, p)]
        ar = O.quantize_act_bf16(io["xb"])
        y_ref, ref_abs = O.gemv_ref(ar, wr)
        assert_gemv_close(eager[(l, p)][:, rows], y_ref, ref_abs, what=f"chain layer {l} proj {p} M={M}")
