"""The accumulation precision of gfx950's FP8 matrix datapath, measured through the library.

Page "02 · DeepGEMM 技术解析" §2.1 explains that an FP8 tensor core sums the products of
one instruction with fewer bits than FP32 (about 14 on Hopper), which is why the method
promotes every 128-long K block into an FP32 accumulator (§2.2).  These tests measure the
same property of the MFMA the library uses: one 128-long K block with unit scales, FP32
output, so D is the matrix unit's own sum of 128 products, compared with the exact float64
block partial of the oracle.  About a million dot products per input distribution.

The ceiling asserted here on adversarial codes is the one the parity gates of
tests/tolerance.py use (EPS_MMA = 2^-11.5 of sum |products|), and 2^-12 on V3-shaped codes;
measured on MI355X over these inputs: 2^-12.0 on every finite code drawn uniformly, 2^-12.2
on random exponent ramps, 2^-12.7 on V3-shaped data.  A datapath that kept the full FP32 sum
would sit near 2^-24.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_amd as dg
import oracle
from tests import gen
from tests.tolerance import EPS_MMA, check_fp32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
M = N = 1024
FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _cases():
    rng = np.random.default_rng(2024)
    p = gen.dense(M, N, 128, seed=7)
    yield "v3", p["a"], p["b"], 2.0 ** -12
    # every finite code equally likely: products spread over ~2^36 of range
    yield "all_codes", rng.choice(FINITE, (M, 128)), rng.choice(FINITE, (N, 128)), EPS_MMA
    # random exponents 1..14 per element, random signs and mantissas
    e, m, s = rng.integers(1, 15, (M, 128)), rng.integers(0, 8, (M, 128)), rng.integers(0, 2, (M, 128))
    yield "exponent_ramps", ((s << 7) | (e << 3) | m).astype(np.uint8), rng.choice(FINITE, (N, 128)), EPS_MMA
    # one dominant product (448 * 448) and 127 small ones of one sign, per row a different gap
    a = np.full((M, 128), 0x30, np.uint8)
    b = np.full((N, 128), 0x30, np.uint8)
    a[:, 0] = b[:, 0] = 0x7E
    for k in range(6):
        a[k::6, 1:] = 0x30 - 8 * k
    a[:, 1:] += rng.integers(0, 8, (M, 127)).astype(np.uint8)
    yield "dominant", a, b, EPS_MMA


@pytest.mark.parametrize("K", [128, 256])
def test_fp8_mfma_block_accumulation_ceiling(K):
    """K = 128 runs the one-block kernel; K = 256 (the block followed by an all-zero block)
    runs the pipelined kernel.  Both must stay under the ceiling."""
    for name, a, b, ceiling in _cases():
        if K == 256:
            a = np.concatenate([a, np.zeros_like(a)], 1)
            b = np.concatenate([b, np.zeros_like(b)], 1)
        sa = np.ones((M, K // 128), np.float32)
        sb = np.ones((N // 128, K // 128), np.float32)
        print("[case] precision", name, K, flush=True)
        d = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        dg.fp8_gemm_nt((torch.from_numpy(a).to(DEV), torch.from_numpy(sa).to(DEV)),
                       (torch.from_numpy(b).to(DEV), torch.from_numpy(sb).to(DEV)), d)
        torch.cuda.synchronize()
        o, T = oracle.gemm_nt(a, sa, b, sb, 128, want_abs=True)
        ok, st = check_fp32(d.cpu().numpy(), o, T, eps=ceiling,
                            name=f"precision one K block, {name} codes, K={K} fp32")
        print("[case] precision", name, K, st, flush=True)
        assert ok.all(), (name, st)
        # and far from a full FP32 sum: the datapath really is narrower (what the per-block
        # promotion guards against)
        if name != "dominant":
            assert st["max_err_over_T"] > 2.0 ** -20, (name, st)
