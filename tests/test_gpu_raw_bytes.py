"""GEMV parity on NVFP4 operands built directly from bytes, not from the
quantizer: every E2M1 code (including 0x8, negative zero) next to every one
of the 254 finite E4M3 block-scale codes (0x00, the subnormals 0x01-0x07,
small and large normals, and the negative codes) on both the weight and the
activation side, with global scales from 2^-20 to 2^4.  The format and the
dequantized value E2M1(code) * E4M3(scale) * global scale are those of the
reading notes, section 2.1; any finite byte pattern, e.g. a caller's own
packed checkpoint, is a valid operand.  Every default kernel variant runs
at M = 1, 2, 4, 8 and 16 (as far as its token count goes), and the LM-head
epilogue runs on the same operands; every output must be within
1e-5 * sum_k |a_k w_k| of the oracle's exact result."""

import numpy as np
import pytest
import torch

import fp4_decode_gemv_amd as F
from oracle import nvfp4_oracle as O
from oracle import reset_oracle as R
from gpu_util import assert_gemv_close

FINITE_E4M3 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)  # 254 codes


def raw_operand(rows: int, K: int, seed: int, gscale: float):
    """codes [rows][K/2], scales [rows][K/16], gscale: every 16-element block
    holds all 16 E2M1 codes once (a per-block rotation of a seeded
    permutation), and the block scales cycle through the 254 finite E4M3
    codes from a seeded offset, so every (code, scale) pair occurs."""
    rng = np.random.default_rng(seed)
    nb = K // 16
    perm = rng.permutation(16).astype(np.uint8)
    rot = (np.arange(rows * nb)[:, None] * 5 + np.arange(16)[None, :]) % 16
    q = perm[rot].reshape(rows, K)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    off = int(rng.integers(0, 254))
    scales = FINITE_E4M3[(np.arange(rows * nb) * 7 + off) % 254].reshape(rows, nb)
    return codes, scales, np.float32(gscale)


def dev_q(t):
    c, s, g = t
    return F.NvFp4Tensor(torch.from_numpy(c).to("cuda:0"), torch.from_numpy(s).to("cuda:0"),
                         torch.tensor([g], dtype=torch.float32, device="cuda:0"))


def test_operands_cover_every_code_and_scale():
    """The construction itself: each E2M1 code appears with each finite
    E4M3 scale on both sides (checked on the host arrays)."""
    for seed in (1, 2):
        c, s, _ = raw_operand(64, 4096, seed, 1.0)
        q = O.unpack_codes(c).reshape(64, -1, 16)
        pairs = set(zip(np.repeat(s.reshape(-1), 16).tolist(), q.reshape(-1).tolist()))
        assert len(pairs) == 254 * 16


GSCALES = [(2.0 ** -20, 2.0 ** 4), (2.0 ** 4, 2.0 ** -20), (1.0, 1.0), (2.0 ** -7, 0.37)]
VARIANTS = F.nvfp4_gemv_variant_names() if __import__("os").path.exists(F.LIB_PATH) else []


@pytest.mark.gpu
@pytest.mark.parametrize("variant", VARIANTS)
def test_every_variant_on_raw_operands(variant):
    mt = F.variant_tokens(variant)
    N, K = 300, 5120
    ran = 0
    with F.forced_variant(variant):
        for M in (1, 2, 4, 8, 16):
            if M > mt:
                continue
            for gi, (ga, gw) in enumerate(GSCALES[:2] if M not in (1, mt) else GSCALES):
                print(f"[raw] {variant} M={M} gA={ga:g} gW={gw:g}", flush=True)
                a = raw_operand(M, K, 10 + M + gi, ga)
                w = raw_operand(N, K, 20 + M + gi, gw)
                if F.nvfp4_gemv_variant(M, N, K) != variant:
                    continue
                y = F.nvfp4_gemv_smallm(dev_q(a), dev_q(w))
                torch.cuda.synchronize()
                y_ref, ref_abs = O.gemv_ref(a, w)
                assert_gemv_close(y.cpu().numpy(), y_ref, ref_abs, what=f"{variant} M={M} gA={ga} gW={gw}")
                ran += 1
    assert ran >= 1, variant


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 2, 8, 16])
def test_lm_head_epilogue_on_raw_operands(M):
    """The LM-head call on byte-built operands: logits against the oracle,
    entropies within 1e-4 nats of the fp64 entropy of the GPU's logits."""
    N, K = 6000, 5120
    a = raw_operand(M, K, 30 + M, 2.0 ** -12)
    w = raw_operand(N, K, 40 + M, 2.0 ** -3)
    dev = torch.device("cuda:0")
    st = F.new_reset_state(M, 8, dev)
    epi = F.Epilogue(step_start=torch.ones(M, dtype=torch.uint8, device=dev), state=st,
                     entropy=torch.empty(M, device=dev), temperature=torch.empty(M, device=dev))
    print(f"[raw lmhead] M={M} N={N} K={K} {F.nvfp4_gemv_variant(M, N, K, True)}", flush=True)
    y = F.nvfp4_gemv_smallm(dev_q(a), dev_q(w), epi=epi)
    torch.cuda.synchronize()
    y_ref, ref_abs = O.gemv_ref(a, w)
    yg = y.cpu().numpy()
    assert_gemv_close(yg, y_ref, ref_abs, what=f"raw lm head M={M}")
    H = epi.entropy.cpu().numpy()
    assert np.all(np.abs(H - R.entropy_rows(yg.astype(np.float64))) <= 1e-4)
    assert np.all(np.abs(H - R.entropy_rows(y_ref)) <= 1e-4)
