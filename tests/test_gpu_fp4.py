"""GPU parity of the FP8 x FP4 GEMMs (FP8 activations, E2M1 weights with one power-of-two scale
per 32 K; page "第13章 DeepGEMM" §13.1 and §13.5) through the C ABI, against the float64
oracle, under the tolerances of tests/tolerance.py."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_amd as dg
import oracle
from tests import gen
from tests.test_gpu_parity import DEV, assert_full_size, bf16_bits, cuda, force_tile, say
from tests.tolerance import check_bf16, check_fp32

pytestmark = pytest.mark.gpu


def _run_dense(p, out=torch.bfloat16, with_c=False, tile=None, c_alias=False):
    d = torch.full((p["M"], p["N"]), float("nan"), dtype=out, device=DEV)
    c = None
    if with_c:
        c = cuda(p["c"])
        if c_alias:
            d.copy_(c)
            c = d
    with force_tile(tile):
        dg.fp8_fp4_gemm_nt((cuda(p["a"]), cuda(p["sa"])), (cuda(p["b"]), cuda(p["sb"])), d, c=c)
    torch.cuda.synchronize()
    return d


def _check(p, d, with_c=False, name=None):
    o, T = oracle.gemm_fp8_fp4_nt(p["a"], p["sa"], p["b"], p["sb"], c=p["c"] if with_c else None, want_abs=True)
    if d.dtype == torch.bfloat16:
        ok, st = check_bf16(bf16_bits(d), o, T, name=name)
    else:
        ok, st = check_fp32(d.cpu().numpy(), o, T, name=name)
    return ok, st


@pytest.mark.parametrize("tile", ["256x224", "128x192"])
@pytest.mark.parametrize("shape", [(200, 300, 384), (257, 513, 256), (33, 129, 640), (64, 32, 1024)])
def test_fp8_fp4_dense_ragged(tile, shape):
    """Every tile, ragged m and n, K from the two-block minimum up, BF16, FP32 and FP32 + C."""
    M, N, K = shape
    p = gen.fp8_fp4(M, N, K, seed=M + N + K, with_c=True)
    for out, with_c in ((torch.bfloat16, False), (torch.float32, False), (torch.float32, True)):
        say("fp8 x fp4 dense", shape, tile, out, with_c)
        d = _run_dense(p, out=out, with_c=with_c, tile=tile)
        ok, st = _check(p, d, with_c=with_c)
        say("fp8 x fp4 dense", st)
        assert ok.all(), (shape, tile, out, with_c, st)


def test_fp8_fp4_c_aliases_d():
    p = gen.fp8_fp4(130, 260, 512, seed=3, with_c=True)
    say("fp8 x fp4 C aliased")
    d1 = _run_dense(p, out=torch.float32, with_c=True)
    d2 = _run_dense(p, out=torch.float32, with_c=True, c_alias=True)
    assert torch.equal(d1, d2)
    ok, st = _check(p, d2, with_c=True)
    assert ok.all(), st


@pytest.mark.parametrize("tile", ["256x224", "128x192"])
def test_fp8_fp4_power_of_two_inputs_are_bitwise_exact(tile):
    """Integer activations in [-2, 2], E2M1 weights up to 2 and power-of-two scales in
    [2^-1, 1]: every partial of 32 or 128 products and their FP32 sum over K = 1024 is exact, so
    FP32 D equals the oracle bitwise and BF16 D is its correct rounding.  The 32-long weight
    scales differ inside each 128-long block, so a scale applied to the wrong K range fails."""
    M, N, K = 150, 260, 1024
    rng = np.random.default_rng(11)
    a = gen.e4m3_codes(rng.integers(-2, 3, (M, K)).astype(np.float32))
    vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0])
    bv = rng.choice(vals, (N, K)) * rng.choice([-1.0, 1.0], (N, K))
    b = gen.pack_fp4(gen.e2m1_codes(bv))
    sa = np.exp2(rng.integers(-1, 1, (M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-1, 1, (N, K // 32))).astype(np.float32)
    p = dict(a=a, sa=sa, b=b, sb=sb, c=None, M=M, N=N, K=K)
    say("fp8 x fp4 exact", tile)
    o = oracle.gemm_fp8_fp4_nt(a, sa, b, sb)
    d = _run_dense(p, out=torch.float32, tile=tile)
    assert np.array_equal(d.cpu().numpy().astype(np.float64), o)
    d = _run_dense(p, out=torch.bfloat16, tile=tile)
    assert np.array_equal(bf16_bits(d), oracle.bf16_rne(o))


def test_fp8_fp4_each_32_block_scale_lands_on_its_k_range():
    """All operands 1.0 except one nonzero 32-long K group per weight row; its scale is 2^t for
    group t, all other groups scaled 2^-20: the result names the group the kernel scaled."""
    M, N, K = 64, 128, 512
    a = np.full((M, K), 0x38, np.uint8)                 # E4M3 1.0
    codes = np.zeros((N, K), np.uint8)
    sub = np.arange(N) % (K // 32)                      # row j: only group sub[j] holds ones
    for j in range(N):
        codes[j, 32 * sub[j]:32 * sub[j] + 32] = 2      # E2M1 1.0
    b = gen.pack_fp4(codes)
    sa = np.ones((M, K // 128), np.float32)
    sb = np.full((N, K // 32), 2.0 ** -20, np.float32)
    sb[np.arange(N), sub] = np.exp2(sub % 8).astype(np.float32)
    p = dict(a=a, sa=sa, b=b, sb=sb, c=None, M=M, N=N, K=K)
    say("fp8 x fp4 scale mapping")
    d = _run_dense(p, out=torch.float32).cpu().numpy()
    want = 32.0 * np.exp2(sub % 8)
    assert np.array_equal(d, np.broadcast_to(want, (M, N)).astype(np.float32))


def test_fp8_fp4_contiguous_ragged():
    """Contiguous groups with FP4 weights: full blocks, a block ending in padding rows, an
    all-padding block, m_total cut inside the last block, a ragged last n tile, sentinels."""
    G, N, K = 4, 300, 512
    p = gen.fp8_fp4_grouped_contiguous(G, N, K, seed=21, m_units=(1, 3))
    starts = np.concatenate([[0], np.cumsum(p["sizes"])])
    layout = p["layout"].copy()
    layout[starts[2] - 40:starts[2]] = -1
    if p["sizes"][2] > 128:
        layout[starts[2]:starts[2] + 128] = -1
    M = p["M"] - 30
    a, sa, layout = p["a"][:M], p["sa"][:M], layout[:M]
    for tile in ("128x256", "128x224"):
        say("fp8 x fp4 contiguous", tile, p["sizes"].tolist(), M)
        d = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        with force_tile(tile):
            dg.m_grouped_fp8_fp4_gemm_nt_contiguous((cuda(a), cuda(sa)), (cuda(p["b"]), cuda(p["sb"])), d,
                                                    cuda(layout))
        torch.cuda.synchronize()
        o, T = oracle.grouped_contiguous_fp8_fp4(a, sa, p["b"], p["sb"], layout, want_abs=True)
        live = ~np.isnan(o)
        ok, st = check_bf16(bf16_bits(d)[live], o[live], T[live])
        say("fp8 x fp4 contiguous", st)
        assert ok.all(), st
        assert np.isnan(d.float().cpu().numpy()[~live]).all()


@pytest.mark.parametrize("tile,K", [("256x224", 256), ("256x224", 768), ("128x224", 384)])
def test_fp8_fp4_masked_ragged(tile, K):
    """Masked groups with FP4 weights: empty, one-row, full and partial groups, ragged n."""
    G, Mmax, N = 5, 256, 500
    p = gen.fp8_fp4_grouped_masked(G, Mmax, N, K, seed=K)
    masked = np.array([0, 256, 1, 129, 200], dtype=np.int32)
    say("fp8 x fp4 masked", tile, K)
    d = torch.full((G, Mmax, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    with force_tile(tile):
        dg.m_grouped_fp8_fp4_gemm_nt_masked((cuda(p["a"]), cuda(p["sa"])), (cuda(p["b"]), cuda(p["sb"])), d,
                                            cuda(masked), expected_m=128)
    torch.cuda.synchronize()
    o, T = oracle.grouped_masked_fp8_fp4(p["a"], p["sa"], p["b"], p["sb"], masked, want_abs=True)
    live = ~np.isnan(o)
    ok, st = check_bf16(bf16_bits(d)[live], o[live], T[live])
    say("fp8 x fp4 masked", st)
    assert ok.all(), st
    assert np.isnan(d.float().cpu().numpy()[~live]).all()


def test_fp8_fp4_dense_full_size_sampled_rows():
    """The dense FP8 x FP4 workload the benchmark times (M = 4096, N = 7168, K = 2048, BF16 out)
    in its launch configuration; rows are independent, so 384 sampled rows (first and last
    included) are checked against the oracle on those rows."""
    p = gen.fp8_fp4(4096, 7168, 2048, seed=0)
    say("fp8 x fp4 dense full size")
    d = _run_dense(p)
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(1).choice(4096, 382, replace=False)]))
    o, T = oracle.gemm_fp8_fp4_nt(p["a"][rows], p["sa"][rows], p["b"], p["sb"], want_abs=True)
    ok, st = check_bf16(bf16_bits(d)[rows], o, T, name=f"fp8 x fp4 dense 4096x7168x2048 ({len(rows)} rows) bf16")
    say("fp8 x fp4 dense full size", st)
    assert ok.all(), st
    assert_full_size(st, "fp8 x fp4 dense")


def test_fp8_fp4_contiguous_full_size_sampled_rows():
    """Contiguous groups with FP4 weights at the size the benchmark times (32 groups of 128 to
    1024 rows, 4096 x 7168 weights), in the planner's launch configuration: the first and last
    row of every group and 8 more rows per group against the oracle."""
    p = gen.fp8_fp4_grouped_contiguous(32, 4096, 7168, seed=0)
    say("fp8 x fp4 contiguous full size", p["M"])
    d = torch.full((p["M"], p["N"]), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.m_grouped_fp8_fp4_gemm_nt_contiguous((cuda(p["a"]), cuda(p["sa"])), (cuda(p["b"]), cuda(p["sb"])), d,
                                            cuda(p["layout"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    starts = np.concatenate([[0], np.cumsum(p["sizes"])])
    rows = np.unique(np.concatenate([np.concatenate([[s, e - 1], rng.integers(s, e, 8)])
                                     for s, e in zip(starts[:-1], starts[1:])]))
    o, T = oracle.grouped_contiguous_fp8_fp4(p["a"][rows], p["sa"][rows], p["b"], p["sb"], p["layout"][rows],
                                             want_abs=True)
    ok, st = check_bf16(bf16_bits(d)[rows], o, T, name=f"fp8 x fp4 contiguous 32x4096x7168 ({len(rows)} rows) bf16")
    say("fp8 x fp4 contiguous full size", st)
    assert ok.all(), st
    assert_full_size(st, "fp8 x fp4 contiguous")


def test_fp8_fp4_masked_full_size_sampled():
    """The masked decode with FP4 weights at the size the benchmark times (32 groups x 256,
    N = 7168, K = 2048): all rows of 4 groups and 32 rows of every other group."""
    p = gen.fp8_fp4_grouped_masked(32, 256, 7168, 2048, seed=0)
    G, Mmax, N = 32, 256, 7168
    say("fp8 x fp4 masked full size", p["masked_m"].tolist())
    d = torch.full((G, Mmax, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.m_grouped_fp8_fp4_gemm_nt_masked((cuda(p["a"]), cuda(p["sa"])), (cuda(p["b"]), cuda(p["sb"])), d,
                                        cuda(p["masked_m"]), expected_m=128)
    torch.cuda.synchronize()
    bits = bf16_bits(d)
    rng = np.random.default_rng(2)
    full = set(rng.choice(G, 4, replace=False).tolist())
    got, os_, Ts = [], [], []
    for g in range(G):
        m = int(p["masked_m"][g])
        if m == 0:
            continue
        rows = np.arange(m) if g in full else np.unique(rng.integers(0, m, 32))
        o, T = oracle.gemm_fp8_fp4_nt(p["a"][g, rows], p["sa"][g, rows], p["b"][g], p["sb"][g], want_abs=True)
        got.append(bits[g, rows]), os_.append(o), Ts.append(T)
    ok, st = check_bf16(np.concatenate(got), np.concatenate(os_), np.concatenate(Ts),
                        name="fp8 x fp4 masked 32x256x7168x2048 (sampled rows) bf16")
    say("fp8 x fp4 masked full size", st)
    assert ok.all(), st
    assert_full_size(st, "fp8 x fp4 masked")
    # rows past masked_m are untouched
    dn = d.float().cpu().numpy()
    for g in range(G):
        assert np.isnan(dn[g, int(p["masked_m"][g]):]).all()
