"""GPU parity: the HIP path (through libdg.so's C ABI) against the float64 oracle
on the same seeded inputs, element by element, under the tolerances in
tests/tolerance.py.  Integer/byte work (the scale transform) is compared bitwise.
Every case prints its name before it touches the GPU."""
import contextlib
import os
import sys

import numpy as np
import pytest
import torch

import block_scaled_fp8_amd as dg
import oracle
from tests import gen
from tests.tolerance import check_bf16, check_fp32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def force_tile(tile):
    old = os.environ.get("DG_FORCE_TILE")
    if tile:
        os.environ["DG_FORCE_TILE"] = tile
    else:
        os.environ.pop("DG_FORCE_TILE", None)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("DG_FORCE_TILE", None)
        else:
            os.environ["DG_FORCE_TILE"] = old


def cuda(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_dense(p, out=torch.bfloat16, tile=None, with_c=False, c_alias=False, recipe=None, pack=False,
              sb_per_row=False):
    M, N = p["M"], p["N"]
    a, b = cuda(p["a"]), cuda(p["b"])
    sa = cuda(p["sa"])
    sb = cuda(p["sb"])
    if sb_per_row:   # weight scales broadcast to one per row (the per-row "1d1d" recipe)
        sb = cuda(oracle.expand_scales_b(p["sb"], N, 128).astype(np.float32))
        recipe = recipe or (1, 1, 128)
    d = torch.full((M, N), float("nan"), dtype=out, device=DEV)
    c = None
    if with_c:
        c = cuda(p["c"])
        if c_alias:
            d.copy_(c)
            c = d
    with force_tile(tile):
        dg.fp8_gemm_nt((a, sa), (b, sb), d, c=c, recipe=recipe, pack_ue8m0=pack)
    torch.cuda.synchronize()
    return d


# Floors and ceilings on the literal-bound statistics of full-size V3-shaped workloads
# (measured on MI355X: FP32 99.1-99.98% within 1e-5 * T and max |d - o| / T 2^-15.5 .. 2^-13.9;
# BF16 99.9988-100% within one ulp or 1e-5 * T).
FULL_FP32_MIN_WITHIN_1E5 = 0.985
FULL_FP32_MAX_ERR = 2.0 ** -12.5
FULL_BF16_MIN_WITHIN = 0.9999


def assert_full_size(st, name):
    if "within_1e5" in st:
        assert st["within_1e5"] >= FULL_FP32_MIN_WITHIN_1E5, (name, st)
        assert st["max_err_over_T"] <= FULL_FP32_MAX_ERR, (name, st)
    else:
        assert st["within_1ulp_or_1e5"] >= FULL_BF16_MIN_WITHIN, (name, st)


def check_dense(p, d, with_c=False, gran_n=128, name="", record=False):
    o, T = oracle.gemm_nt(p["a"], p["sa"], p["b"], p["sb"], 128, c=p["c"] if with_c else None, want_abs=True)
    rec = name if record else None
    if d.dtype == torch.bfloat16:
        ok, st = check_bf16(bf16_bits(d), o, T, name=rec)
    else:
        ok, st = check_fp32(d.cpu().numpy(), o, T, name=rec)
    say(name, st)
    assert ok.all(), (name, st)
    return st


# ---------------------------------------------------------------- transform (bitwise)
@pytest.mark.parametrize("G,mn,sf_k,gran", [(1, 6, 5, 1), (1, 4096, 16, 1), (3, 37, 7, 1), (2, 300, 56, 128),
                                            (32, 7168, 16, 128), (1, 1, 1, 1)])
@pytest.mark.parametrize("pack", [False, True])
def test_transform_matches_oracle_bitwise(G, mn, sf_k, gran, pack):
    say("transform", G, mn, sf_k, gran, pack)
    rng = np.random.default_rng(G * 1000 + mn + sf_k)
    mnb = (mn + gran - 1) // gran
    sf = (rng.random((G, mnb, sf_k)) * 4 + 1e-3).astype(np.float32)
    sf[..., ::3] = np.exp2(rng.integers(-10, 5, size=sf[..., ::3].shape)).astype(np.float32)
    ref, cnt = oracle.transform_sf(sf, mn, gran, pack)
    count = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = dg.transform_sf(cuda(sf), mn, gran, pack, nonpow2_count=count)
    torch.cuda.synchronize()
    # the whole underlying buffer, padding rows included
    a4 = (mn + 3) // 4 * 4
    cols = out.shape[-1]
    raw = torch.as_strided(out, (G, cols, a4), (cols * a4, a4, 1)).cpu().numpy()
    assert raw.dtype == ref.dtype
    assert np.array_equal(raw.view(np.uint32), ref.reshape(G, cols, a4).view(np.uint32))
    if pack:
        assert int(count.item()) == cnt


def test_transform_page_examples():
    # 0.75 -> UE8M0 0.5 (code 126), 3 -> 2 (code 128); both counted as non-powers of two
    say("transform page examples")
    sf = np.array([[0.75, 3.0, 1.0, 0.5]], dtype=np.float32)
    count = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = dg.transform_sf(cuda(sf), 1, 1, True, nonpow2_count=count)
    w = int(out.cpu().numpy().view(np.uint32)[0, 0])
    assert [(w >> (8 * t)) & 0xFF for t in range(4)] == [126, 128, 127, 126]
    assert int(count.item()) == 2


# ---------------------------------------------------------------- per-token-group cast (bitwise)
def _cast_input(m, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    n = max(1, (m * k) // 1000)
    x.reshape(-1)[rng.choice(m * k, size=n, replace=False)] *= np.float32(50.0)   # outliers
    x[0, :128] = 0.0                                                            # an all-zero group
    if k >= 256:
        # amax 448 makes the scale 1, so these quotients sit exactly on E4M3 rounding ties
        pos = np.sort(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
        mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
        row = np.resize(np.concatenate([mids, -mids]), 128)
        row[0] = 448.0
        x[-1, 128:256] = row
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m,k", [(1, 128), (3, 384), (5, 640), (37, 1152), (130, 7168)])
def test_per_token_group_cast_bitwise(dtype, m, k):
    """Codes and scales of the per-token-group cast against the oracle, bit for bit.  The rows
    mix N(0,1) values, x50 outliers, an all-zero group and exact rounding ties; k/128 not a
    multiple of 4 leaves the last wave of each row partly idle."""
    x = _cast_input(m, k, seed=m * 7 + k)
    say("cast", dtype, m, k)
    xt = torch.from_numpy(x).to(DEV).to(dtype)
    q, sf = dg.per_token_group_cast_fp8(xt)
    torch.cuda.synchronize()
    seen = xt.float().cpu().numpy()          # the values the kernel read (BF16-rounded for BF16)
    qo, so = oracle.per_token_group_cast(seen)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), so.view(np.uint32))


def test_cast_feeds_the_gemm():
    """The cast's outputs are the GEMM's A operand and activation scales as they stand."""
    p = gen.dense(200, 384, 512, seed=41)
    x = _cast_input(200, 512, seed=42)
    say("cast -> gemm")
    q, sf = dg.per_token_group_cast_fp8(torch.from_numpy(x).to(DEV))
    d = torch.full((200, 384), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.fp8_gemm_nt((q, sf), (cuda(p["b"]), cuda(p["sb"])), d)
    torch.cuda.synchronize()
    qo, so = oracle.per_token_group_cast(x)
    o, T = oracle.gemm_nt(qo, so, p["b"], p["sb"], 128, want_abs=True)
    ok, st = check_bf16(bf16_bits(d), o, T)
    say("cast -> gemm", st)
    assert ok.all(), st


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m,k", [(1, 128), (3, 384), (5, 640), (9, 1664), (37, 1152), (130, 7168)])
def test_per_token_group_cast_ue8m0_bitwise(dtype, m, k):
    """The cast with power-of-two scales: E4M3 codes bit for bit against the oracle, and the
    packed scale words against the oracle's own packing of its scales (k/128 = 1, 3, 5, 13,
    9, 56 groups: one, partly and exactly filled last words)."""
    x = _cast_input(m, k, seed=m * 11 + k)
    say("cast ue8m0", dtype, m, k)
    xt = torch.from_numpy(x).to(DEV).to(dtype)
    q, sf = dg.per_token_group_cast_fp8(xt, pack_ue8m0=True)
    torch.cuda.synchronize()
    seen = xt.float().cpu().numpy()
    qo, so = oracle.per_token_group_cast(seen, ue8m0=True)
    words, _ = oracle.transform_sf(so, m, 1, True)            # [ceil(sf_k/4), align4(m)]
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), words[:, :m].T.view(np.uint32))


@pytest.mark.parametrize("pack", [False, True])
def test_cast_out_overwrites_an_earlier_result(pack):
    """``out=`` reuses the buffers of an earlier call on a smaller-valued input: every code and
    scale is rewritten (no stale value from the first call survives)."""
    x1, x2 = _cast_input(70, 640, seed=3), _cast_input(70, 640, seed=4) * np.float32(0.01)
    say("cast out=", pack)
    first = dg.per_token_group_cast_fp8(torch.from_numpy(x1).to(DEV), pack_ue8m0=pack)
    q, sf = dg.per_token_group_cast_fp8(torch.from_numpy(x2).to(DEV), pack_ue8m0=pack, out=first)
    fresh_q, fresh_sf = dg.per_token_group_cast_fp8(torch.from_numpy(x2).to(DEV), pack_ue8m0=pack)
    torch.cuda.synchronize()
    assert q.data_ptr() == first[0].data_ptr() and sf.data_ptr() == first[1].data_ptr()
    assert torch.equal(q.cpu(), fresh_q.cpu())
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), fresh_sf.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("pack", [False, True])
def test_cast_full_size_sampled_rows(pack):
    """The cast at the size the benchmark times (4096 x 7168 BF16), in the same launch
    configuration; rows are cast independently, so 66 sampled rows (first and last included)
    are checked bit for bit against the oracle run on those rows."""
    m, k = 4096, 7168
    x = _cast_input(m, k, seed=77)
    say("cast full size", pack)
    xt = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    q, sf = dg.per_token_group_cast_fp8(xt, pack_ue8m0=pack)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(78).integers(0, m, 64)]))
    seen = xt[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    qo, so = oracle.per_token_group_cast(seen, ue8m0=pack)
    assert np.array_equal(q.cpu().numpy()[rows], qo)
    got = sf.cpu().numpy()[rows].view(np.uint32)
    if pack:
        words, _ = oracle.transform_sf(so, len(rows), 1, True)
        assert np.array_equal(got, words[:, :len(rows)].T.view(np.uint32))
    else:
        assert np.array_equal(got, so.view(np.uint32))


def test_cast_ue8m0_feeds_the_gemm():
    """Packed UE8M0 output of the cast is the GEMM's activation scale operand as it stands."""
    p = gen.grouped_masked(1, 200, 384, 640, seed=43, pow2_scales=True)
    x = _cast_input(200, 640, seed=44)
    say("cast ue8m0 -> gemm")
    q, sf = dg.per_token_group_cast_fp8(torch.from_numpy(x).to(DEV), pack_ue8m0=True)
    sb = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(cuda(p["sb"][0]), gran_mn=128, mn=384)
    d = torch.full((200, 384), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.fp8_gemm_nt((q, sf), (cuda(p["b"][0]), sb), d)
    torch.cuda.synchronize()
    qo, so = oracle.per_token_group_cast(x, ue8m0=True)
    o, T = oracle.gemm_nt(qo, so, p["b"][0], p["sb"][0], 128, want_abs=True)
    ok, st = check_bf16(bf16_bits(d), o, T)
    say("cast ue8m0 -> gemm", st)
    assert ok.all(), st


# ---------------------------------------------------------------- K-grouped
@pytest.mark.parametrize("alias", [True, False])
@pytest.mark.parametrize("m,n,ks", [(260, 196, [256, 0, 384, 128, 512]), (64, 520, [128]), (4, 4, [0, 128, 0]),
                                    (516, 388, [1024, 128, 0, 640])])
def test_k_grouped_contiguous(m, n, ks, alias):
    """K-grouped GEMM against the oracle: groups of 1 to 8 K blocks and empty groups (D = C),
    m and n ragged against every tile, C read separately or accumulated in place in D."""
    p = gen.k_grouped(m, n, ks, seed=m + n + len(ks))
    say("k-grouped", m, n, ks, "alias" if alias else "separate C")
    a, b = cuda(p["a"]), cuda(p["b"])
    sfa, sfb = cuda(np.ascontiguousarray(p["sa"].T)), cuda(np.ascontiguousarray(p["sb"].T))
    c = cuda(p["c"])
    if alias:
        d = c.clone()
        dg.k_grouped_fp8_gemm_nt_contiguous((a, sfa), (b, sfb), d, ks, d)
    else:
        d = torch.full_like(c, float("nan"))
        dg.k_grouped_fp8_gemm_nt_contiguous((a, sfa), (b, sfb), d, ks, c)
    torch.cuda.synchronize()
    o, T = oracle.k_grouped(p["a"], p["sa"], p["b"], p["sb"], ks, p["c"], want_abs=True)
    got = d.cpu().numpy()
    ok, st = check_fp32(got, o, T)
    say("k-grouped", st)
    assert ok.all(), st
    for g, k in enumerate(ks):
        if k == 0:
            assert np.array_equal(got[g], p["c"][g])      # an empty group is C, bit for bit
    if not alias:
        assert torch.equal(c.cpu(), torch.from_numpy(p["c"]))   # C is only read


def test_k_grouped_full_size_sampled():
    """The K-grouped weight-gradient workload at the size the benchmark times (m = 7168,
    n = 2048, eight groups, K = 16384 in all), accumulated in place as the benchmark runs it,
    checked on 1024 sampled outputs per group against the oracle evaluated point by point."""
    ks = [1792, 2304, 2048, 1536, 2560, 2048, 1920, 2176]
    m, n = 7168, 2048
    p = gen.k_grouped(m, n, ks, seed=9)
    say("k-grouped full size", m, n, ks)
    d = cuda(p["c"])
    dg.k_grouped_fp8_gemm_nt_contiguous((cuda(p["a"]), cuda(np.ascontiguousarray(p["sa"].T))),
                                        (cuda(p["b"]), cuda(np.ascontiguousarray(p["sb"].T))), d, ks, d)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    rng = np.random.default_rng(10)
    k0 = 0
    allo, allT, alld = [], [], []
    for g, k in enumerate(ks):
        ii, jj = rng.integers(0, m, 1024), rng.integers(0, n, 1024)
        ii[:2], jj[:2] = [0, m - 1], [0, n - 1]                       # the corners
        kr, br = slice(k0, k0 + k), slice(k0 // 128, (k0 + k) // 128)
        o, T = oracle.gemm_nt_points(p["a"][:, kr], p["sa"][:, br], p["b"][:, kr], p["sb"][:, br], ii, jj, 1,
                                     c=p["c"][g])
        ok, st = check_fp32(got[g][ii, jj], o, T)
        say("k-grouped full size group", g, st)
        assert ok.all(), (g, st)
        allo.append(o); allT.append(T); alld.append(got[g][ii, jj])
        k0 += k
    ok, st = check_fp32(np.concatenate(alld), np.concatenate(allo), np.concatenate(allT),
                        name="k-grouped 8x7168x2048 k16384 fp32 (8192 sampled)")
    # both operands are activation-like (x50 outliers on both sides): measured 98-99% within 1e-5 * T
    assert st["within_1e5"] >= 0.97 and st["max_err_over_T"] <= FULL_FP32_MAX_ERR, st


# ---------------------------------------------------------------- dense
def test_config1_tiny_bf16():
    p = gen.config1()
    say("config1 tiny", p["M"], p["N"], p["K"])
    d = run_dense(p)
    st = check_dense(p, d, name="config1 128x256x512 bf16", record=True)
    assert st["within_1ulp_or_1e5"] == 1.0, st


DENSE_TILES = ["256x224", "256x256", "128x224", "128x256", "128x128", "64x128", "128x192", "256x192", "64x32"]


@pytest.mark.parametrize("tile", DENSE_TILES)
@pytest.mark.parametrize("shape", [(200, 300, 384), (257, 513, 256), (33, 129, 640)])
def test_dense_ragged_every_tile(tile, shape):
    M, N, K = shape
    p = gen.dense(M, N, K, seed=M + N + K)
    say("dense ragged", shape, tile)
    d = run_dense(p, out=torch.bfloat16, tile=tile)
    check_dense(p, d, name=f"dense bf16 {shape} {tile}")
    d32 = run_dense(p, out=torch.float32, tile=tile)
    check_dense(p, d32, name=f"dense f32 {shape} {tile}")


@pytest.mark.parametrize("tile", ["256x224", "128x192", "128x128", "64x32"])
def test_pow2_inputs_are_bitwise_exact(tile):
    # integer payloads and power-of-two scales: every FP32 partial sum is exact, so the
    # FP32 result equals the oracle bitwise and BF16 is its correct rounding
    p = gen.pow2_exact(300, 520, 1024, seed=3, with_c=True)
    say("pow2 exact", tile)
    o = oracle.gemm_nt(p["a"], p["sa"], p["b"], p["sb"], 128, c=p["c"])
    d = run_dense(p, out=torch.float32, tile=tile, with_c=True)
    assert np.array_equal(d.cpu().numpy().astype(np.float64), o)
    o0 = oracle.gemm_nt(p["a"], p["sa"], p["b"], p["sb"], 128)
    d = run_dense(p, out=torch.bfloat16, tile=tile)
    assert np.array_equal(bf16_bits(d), oracle.bf16_rne(o0))


@pytest.mark.parametrize("tile", ["256x224", "128x192"])
def test_ue8m0_long_k_accumulation_is_fp32_exact(tile):
    """UE8M0 scales: the scaled MFMA adds every block's product into the FP32 accumulator.
    Integer payloads in [-8, 8] and scales 2^e, e in [-3, 0], over K = 4096 (32 blocks): every
    partial sum fits 24 significant bits, so an FP32 accumulation is exact and the result must
    equal the oracle bitwise.  An accumulator narrower than FP32 (the concern the pages raise
    for FP8 tensor cores, which is why they promote every 128) would round typical sums of
    about 15 significant bits."""
    p = gen.pow2_exact(300, 520, 4096, seed=21)
    say("ue8m0 long-K exact", tile)
    o = oracle.gemm_nt(p["a"], p["sa"], p["b"], p["sb"], 128)
    d = run_dense(p, out=torch.float32, tile=tile, pack=True, sb_per_row=True)
    assert np.array_equal(d.cpu().numpy().astype(np.float64), o)
    d = run_dense(p, out=torch.bfloat16, tile=tile, pack=True, sb_per_row=True)
    assert np.array_equal(bf16_bits(d), oracle.bf16_rne(o))


def test_c_accumulation_and_aliasing():
    p = gen.dense(256, 384, 512, seed=4, with_c=True)
    say("C accumulation")
    d = run_dense(p, out=torch.float32, with_c=True)
    check_dense(p, d, with_c=True, name="C separate")
    d2 = run_dense(p, out=torch.float32, with_c=True, c_alias=True)
    check_dense(p, d2, with_c=True, name="C aliased")
    assert torch.equal(d, d2)


def test_straddling_tiles_equal_aligned_tiles_bitwise():
    # the same problem with N tiles that straddle 128-wide weight-scale blocks (224, 192)
    # and tiles that do not (128, 256): each output element sees the same MFMA and the same
    # promotion order, so the results are identical
    p = gen.dense(512, 1536, 1024, seed=5, with_c=True)
    say("straddle vs aligned")
    outs = {t: run_dense(p, out=torch.float32, tile=t, with_c=True).cpu() for t in
            ["128x128", "256x256", "256x224", "128x192", "256x192", "128x224", "64x32"]}
    check_dense(p, outs["256x224"].to(DEV), with_c=True, name="straddle 256x224")
    ref = outs["128x128"]
    for t, v in outs.items():
        assert torch.equal(v, ref), t


@pytest.mark.parametrize("pack", [False, True])
def test_per_row_weight_scales(pack):
    # recipe (1, 1, 128): weight scales broadcast per row, FP32 or packed UE8M0
    p = gen.grouped_masked(1, 300, 520, 768, seed=6, pow2_scales=True)
    q = dict(a=p["a"][0], sa=p["sa"][0], b=p["b"][0], sb=p["sb"][0], c=None, M=300, N=520, K=768)
    say("per-row weight scales", pack)
    d = run_dense(q, out=torch.float32, sb_per_row=True, pack=pack)
    check_dense(q, d, name=f"1d1d pack={pack}")
    d2 = run_dense(q, out=torch.float32)
    check_dense(q, d2, name="1d2d same data")


@pytest.mark.parametrize("tile", ["256x224", "128x192"])
@pytest.mark.parametrize("out", ["bf16", "f32", "f32+c"])
def test_pipelined_per_row_fp32_weight_scales(tile, out):
    """FP32 per-row weight scales on the pipelined tiles: every weight row has its own scale
    per K block (so a lane that read a neighbouring column's scale would fail), ragged m and
    n, K from the minimum two blocks up, BF16, FP32 and FP32 + C output."""
    for M, N, K in [(300, 520, 512), (37, 200, 256)]:
        p = gen.dense(M, N, K, seed=M + K, with_c=out == "f32+c")
        rng = np.random.default_rng(M + N)
        sb = rng.uniform(0.002, 0.03, (N, K // 128)).astype(np.float32)
        say("pipelined 1d1d fp32", tile, out, M, N, K)
        c = cuda(p["c"]) if out == "f32+c" else None
        d = torch.full((M, N), float("nan"), dtype=torch.bfloat16 if out == "bf16" else torch.float32, device=DEV)
        with force_tile(tile):
            dg.fp8_gemm_nt((cuda(p["a"]), cuda(p["sa"])), (cuda(p["b"]), cuda(sb)), d, c=c, recipe=(1, 1, 128))
        torch.cuda.synchronize()
        o, T = oracle.gemm_nt(p["a"], p["sa"], p["b"], sb, 1, c=p["c"] if c is not None else None, want_abs=True)
        if out == "bf16":
            ok, st = check_bf16(bf16_bits(d), o, T)
        else:
            ok, st = check_fp32(d.cpu().numpy(), o, T)
        say("pipelined 1d1d fp32", st)
        assert ok.all(), st


def test_deterministic_and_batch_invariant():
    p = gen.dense(1024, 768, 1024, seed=7)
    say("determinism / batch invariance")
    d1 = run_dense(p, tile="128x128")
    d2 = run_dense(p, tile="128x128")
    assert torch.equal(d1, d2)
    q = dict(p, a=p["a"][:64], sa=p["sa"][:64], M=64)
    d3 = run_dense(q, tile="128x128")
    assert torch.equal(d3, d1[:64])


def test_empty_and_tiny_problems():
    say("empty / tiny")
    p = gen.dense(1, 8, 128, seed=8)
    d = run_dense(p)
    check_dense(p, d, name="1x8x128")
    a = torch.zeros((0, 256), dtype=torch.uint8, device=DEV)
    sa = torch.zeros((0, 2), dtype=torch.float32, device=DEV)
    b = torch.zeros((64, 256), dtype=torch.uint8, device=DEV)
    sb = torch.ones((1, 2), dtype=torch.float32, device=DEV)
    d = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    dg.fp8_gemm_nt((a, sa), (b, sb), d)
    torch.cuda.synchronize()


def test_sentinel_coverage_ragged():
    # every valid element written exactly where it belongs; the padding of a strided D untouched
    p = gen.dense(130, 200, 256, seed=9)
    say("sentinel coverage")
    a, b, sa, sb = cuda(p["a"]), cuda(p["b"]), cuda(p["sa"]), cuda(p["sb"])
    big = torch.full((130, 264), -12345.0, dtype=torch.float32, device=DEV)
    d = big[:, :200]
    dg.fp8_gemm_nt((a, sa), (b, sb), d)
    torch.cuda.synchronize()
    h = big.cpu().numpy()
    assert (h[:, 200:] == -12345.0).all()
    o, T = oracle.gemm_nt(p["a"], p["sa"], p["b"], p["sb"], 128, want_abs=True)
    ok, st = check_fp32(h[:, :200], o, T)
    assert ok.all(), st


# ---------------------------------------------------------------- grouped (small)
def test_contiguous_small_with_padding_rows():
    G, N, K = 4, 384, 512
    p = gen.grouped_contiguous(G, N, K, seed=10, m_units=(1, 3))
    layout = p["layout"].copy()
    # pad the last 60 rows of group 1's segment: they must not be written
    seg = np.nonzero(layout == 1)[0]
    layout[seg[-60:]] = -1
    say("contiguous small", p["sizes"])
    a, sa = cuda(p["a"]), cuda(p["sa"])
    b, sb = cuda(p["b"]), cuda(p["sb"])
    d = torch.full((p["M"], N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.m_grouped_fp8_gemm_nt_contiguous((a, sa), (b, sb), d, cuda(layout))
    torch.cuda.synchronize()
    o, T = oracle.grouped_contiguous(p["a"], p["sa"], p["b"], p["sb"], layout, want_abs=True)
    bits = bf16_bits(d)
    live = layout >= 0
    ok, st = check_bf16(bits[live], o[live], T[live])
    say("contiguous small", st)
    assert ok.all(), st
    assert np.isnan(d.float().cpu().numpy()[~live]).all()


@contextlib.contextmanager
def grid_size(n):
    if n:
        dg.set_num_sms(n)
    try:
        yield
    finally:
        if n:
            dg.set_num_sms(0)


def pow2_floor(s):
    """Largest power of two <= each (positive, normal) scale: inputs that UE8M0 holds exactly."""
    return np.exp2(np.floor(np.log2(s))).astype(np.float32)


@pytest.mark.parametrize("tile,out,pack,sms,K", [("128x256", torch.bfloat16, False, None, 768),
                                                 ("128x256", torch.bfloat16, False, 5, 768),
                                                 ("128x224", torch.float32, False, 3, 768),
                                                 ("128x224", torch.bfloat16, True, 5, 768),
                                                 ("128x256", torch.bfloat16, True, None, 768),
                                                 ("128x256", torch.bfloat16, False, 5, 256)])
def test_contiguous_pipelined_ragged(tile, out, pack, sms, K):
    """Contiguous groups on the pipelined tiles: full blocks, a block ending in padding rows
    (rows checked one by one), a block that is all padding and one naming no group (both
    skipped), m_total cut short inside the last block, a ragged last n tile; a small grid
    makes every workgroup walk several tiles across those cases.  K = 256 is the pipelined
    kernel's minimum: two K blocks, so every copy a block issues is for the next tile."""
    G, N = 5, 500
    p = gen.grouped_contiguous(G, N, K, seed=16, m_units=(1, 3))
    starts = np.concatenate([[0], np.cumsum(p["sizes"])])
    assert list(p["sizes"]) == [256, 256, 384, 256, 384]
    layout = p["layout"].copy()
    layout[starts[2] - 60:starts[2]] = -1          # group 1 ends in 60 padding rows
    layout[starts[2]:starts[2] + 128] = -1         # group 2's first block is all padding
    layout[starts[3]:starts[3] + 128] = G + 2      # a block naming no group
    M = p["M"] - 50                                # the last block has 78 rows
    a, sa, layout = p["a"][:M], p["sa"][:M], layout[:M]
    sb = p["sb"]
    if pack:
        sa, sb = pow2_floor(sa), pow2_floor(sb)
    say("contiguous pipelined", tile, out, pack, sms, K, M)
    d = torch.full((M, N), float("nan"), dtype=out, device=DEV)
    with force_tile(tile), grid_size(sms):
        dg.m_grouped_fp8_gemm_nt_contiguous((cuda(a), cuda(sa)), (cuda(p["b"]), cuda(sb)), d, cuda(layout),
                                            pack_ue8m0=pack)
    torch.cuda.synchronize()
    o, T = oracle.grouped_contiguous(a, sa, p["b"], sb, layout, want_abs=True)
    live = ~np.isnan(o)
    assert live.sum() == (M - 60 - 256) * N
    if out == torch.bfloat16:
        ok, st = check_bf16(bf16_bits(d)[live], o[live], T[live])
    else:
        ok, st = check_fp32(d.cpu().numpy()[live], o[live], T[live])
    say("contiguous pipelined", st)
    assert ok.all(), st
    assert np.isnan(d.float().cpu().numpy()[~live]).all()


@pytest.mark.parametrize("tile", [None, "128x128", "256x224", "64x32"])
def test_masked_small_with_sentinels(tile):
    G, Mmax, N, K = 5, 200, 300, 256
    p = gen.grouped_masked(G, Mmax, N, K, seed=11, pow2_scales=False)
    masked = np.array([0, 200, 1, 129, 77], dtype=np.int32)
    say("masked small", tile, masked)
    a, sa = cuda(p["a"]), cuda(p["sa"])
    b, sb = cuda(p["b"]), cuda(p["sb"])
    d = torch.full((G, Mmax, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    with force_tile(tile):
        dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, cuda(masked), expected_m=100)
    torch.cuda.synchronize()
    o, T = oracle.grouped_masked(p["a"], p["sa"], p["b"], p["sb"], masked, want_abs=True)
    bits = bf16_bits(d)
    live = ~np.isnan(o)
    ok, st = check_bf16(bits[live], o[live], T[live])
    say("masked small", st)
    assert ok.all(), st
    assert np.isnan(d.float().cpu().numpy()[~live]).all()


@pytest.mark.parametrize("tile,pack,K", [("128x224", False, 768), ("128x224", True, 768), ("128x224", True, 384),
                                         ("256x224", False, 768), ("256x224", True, 768), ("256x224", True, 256)])
def test_masked_pipelined_ragged(tile, pack, K):
    """Masked groups on the pipelined tiles (128 rows with three B stages, 256 rows with two):
    empty, one-row, full, straddling and exact-multiple groups, a ragged last n tile, and
    (pack) UE8M0 scales applied inside the MFMA."""
    # (K = 384: exactly as many K blocks as B stages, so every prefetch crosses into the next tile)
    G, Mmax, N = 6, 300, 500
    p = gen.grouped_masked(G, Mmax, N, K, seed=12, pow2_scales=pack)
    masked = np.array([0, 300, 1, 129, 255, 128], dtype=np.int32)
    say("masked pipelined", tile, pack, K, masked)
    a, b = cuda(p["a"]), cuda(p["b"])
    if pack:
        sa = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(cuda(p["sa"]))
        sb = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(cuda(p["sb"]), gran_mn=128, mn=N)
    else:
        sa, sb = cuda(p["sa"]), cuda(p["sb"])
    d = torch.full((G, Mmax, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    with force_tile(tile):
        dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, cuda(masked), expected_m=128)
    torch.cuda.synchronize()
    o, T = oracle.grouped_masked(p["a"], p["sa"], p["b"], p["sb"], masked, want_abs=True)
    bits = bf16_bits(d)
    live = ~np.isnan(o)
    ok, st = check_bf16(bits[live], o[live], T[live])
    say("masked pipelined", st)
    assert ok.all(), st
    assert np.isnan(d.float().cpu().numpy()[~live]).all()


# ---------------------------------------------------------------- the five workloads at full size
def test_config2_dense_full():
    p = gen.config2()
    say("config2 4096x7168x2048 bf16")
    d = run_dense(p)
    st = check_dense(p, d, name="config2 4096x7168x2048 bf16", record=True)
    assert_full_size(st, "config2")
    d32 = run_dense(p, out=torch.float32)
    st = check_dense(p, d32, name="config2 4096x7168x2048 fp32", record=True)
    assert_full_size(st, "config2 fp32")


def test_config2_decode_m64_full():
    p = gen.config2(M=64)
    say("config2 M=64")
    d = run_dense(p)
    st = check_dense(p, d, name="config2 64x7168x2048 bf16", record=True)
    assert_full_size(st, "config2 M64")
    d32 = run_dense(p, out=torch.float32)
    st = check_dense(p, d32, name="config2 64x7168x2048 fp32", record=True)
    assert_full_size(st, "config2 M64 fp32")


def test_config3_1d2d_with_c_full():
    p = gen.config3()
    say("config3 4096x1536x7168 f32 + C")
    d = run_dense(p, out=torch.float32, with_c=True)
    st = check_dense(p, d, with_c=True, name="config3 4096x1536x7168 fp32+C", record=True)
    assert_full_size(st, "config3")
    bm, bn, _, _ = dg.get_gemm_config(0, 4096, 1536, 7168, d_dtype=2, num_sms=dg.get_num_sms())
    say("config3 tile", bm, bn)


def test_config4_contiguous_sampled_rows():
    p = gen.config4()
    G, N = p["G"], p["N"]
    say("config4 contiguous", p["M"], "rows")
    a, sa = cuda(p["a"]), cuda(p["sa"])
    b, sb = cuda(p["b"]), cuda(p["sb"])
    d = torch.full((p["M"], N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.m_grouped_fp8_gemm_nt_contiguous((a, sa), (b, sb), d, cuda(p["layout"]))
    torch.cuda.synchronize()
    bits = bf16_bits(d)
    assert not np.isnan(d.float().cpu().numpy()).any()
    # all rows of 4 groups and 64 random rows of every other group
    rng = np.random.default_rng(123)
    starts = np.concatenate([[0], np.cumsum(p["sizes"])])
    full = set(rng.choice(G, 4, replace=False).tolist())
    rows = []
    for g in range(G):
        seg = np.arange(starts[g], starts[g + 1])
        rows.append(seg if g in full else rng.choice(seg, 64, replace=False))
    rows = np.sort(np.concatenate(rows))
    sub_layout = p["layout"][rows]
    o, T = oracle.grouped_contiguous(p["a"][rows], p["sa"][rows], p["b"], p["sb"], sub_layout, want_abs=True)
    ok, st = check_bf16(bits[rows], o, T, name=f"config4 contiguous 32x4096x7168 ({len(rows)} rows) bf16")
    say("config4", len(rows), "rows", st)
    assert ok.all(), st
    assert_full_size(st, "config4")


def test_config5_masked_full_with_sentinels():
    p = gen.config5()
    G, Mmax, N = p["G"], p["M_max"], p["N"]
    say("config5 masked", p["masked_m"].tolist())
    a, b = cuda(p["a"]), cuda(p["b"])
    sa = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(cuda(p["sa"]))
    sb = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(cuda(p["sb"]), gran_mn=128, mn=N)
    d = torch.full((G, Mmax, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, cuda(p["masked_m"]), expected_m=128)
    torch.cuda.synchronize()
    o, T = oracle.grouped_masked(p["a"], p["sa"], p["b"], p["sb"], p["masked_m"], want_abs=True)
    bits = bf16_bits(d)
    live = ~np.isnan(o)
    ok, st = check_bf16(bits[live], o[live], T[live], name="config5 masked 32x256x7168x2048 bf16")
    say("config5", st)
    assert ok.all(), st
    assert_full_size(st, "config5")
    assert np.isnan(d.float().cpu().numpy()[~live]).all()


# ---------------------------------------------------------------- contract edges
@pytest.mark.parametrize("tile,K", [("128x224", 384), ("256x224", 256)])
def test_masked_more_than_64_groups(tile, K):
    """More groups than a wave has lanes: the tile walk over groups takes its serial path
    (one scalar read of masked_m per group).  Empty, full and partial groups, sentinels."""
    G, Mmax, N = 70, 64, 260
    p = gen.grouped_masked(G, Mmax, N, K, seed=G + K, pow2_scales=False)
    masked = np.random.default_rng(5).integers(0, Mmax + 1, G).astype(np.int32)
    masked[[0, 33, 64, 69]] = [0, Mmax, 1, Mmax]
    say("masked > 64 groups", tile, K)
    d = torch.full((G, Mmax, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    with force_tile(tile):
        dg.m_grouped_fp8_gemm_nt_masked((cuda(p["a"]), cuda(p["sa"])), (cuda(p["b"]), cuda(p["sb"])), d,
                                        cuda(masked), expected_m=32)
    torch.cuda.synchronize()
    o, T = oracle.grouped_masked(p["a"], p["sa"], p["b"], p["sb"], masked, want_abs=True)
    live = ~np.isnan(o)
    ok, st = check_bf16(bf16_bits(d)[live], o[live], T[live])
    say("masked > 64 groups", st)
    assert ok.all(), st
    assert np.isnan(d.float().cpu().numpy()[~live]).all()


def test_masked_graph_capture_and_replay():
    """The masked layout exists so the call can sit in a captured graph with static shapes
    (page "02 · DeepGEMM 技术解析" §5.2): captured once, replayed with new masked_m contents
    written between replays; every replay matches the oracle and leaves masked rows alone."""
    G, Mmax, N, K = 6, 200, 300, 512
    p = gen.grouped_masked(G, Mmax, N, K, seed=31, pow2_scales=True)
    say("masked graph capture")
    a, b = cuda(p["a"]), cuda(p["b"])
    sa = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(cuda(p["sa"]))
    sb = dg.get_mn_major_tma_aligned_packed_ue8m0_tensor(cuda(p["sb"]), gran_mn=128, mn=N)
    mm = torch.zeros(G, dtype=torch.int32, device=DEV)
    d = torch.full((G, Mmax, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, mm, expected_m=128)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, mm, expected_m=128)
    for masks in ([0, 200, 1, 129, 77, 64], [200, 0, 0, 5, 128, 199], [3, 3, 3, 3, 3, 3], [0, 200, 1, 129, 77, 64]):
        m = np.array(masks, dtype=np.int32)
        mm.copy_(torch.from_numpy(m).to(DEV))
        d.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o, T = oracle.grouped_masked(p["a"], p["sa"], p["b"], p["sb"], m, want_abs=True)
        live = ~np.isnan(o)
        ok, st = check_bf16(bf16_bits(d)[live], o[live], T[live])
        say("masked graph replay", masks, st)
        assert ok.all(), (masks, st)
        assert np.isnan(d.float().cpu().numpy()[~live]).all()


@pytest.mark.parametrize("pack", [False, True])
def test_raw_block_weight_scales_small_n(pack):
    """Raw 128x128 weight scales of a weight matrix with n <= 128 rows (one block row),
    broadcast per row by the binding: FP32 per-row scales and packed UE8M0."""
    M, N, K = 70, 100, 512
    p = gen.dense(M, N, K, seed=17)
    sa, sb = pow2_floor(p["sa"]), pow2_floor(p["sb"])
    assert sb.shape == (1, K // 128)
    say("small-n raw block scales", pack)
    d = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    dg.fp8_gemm_nt((cuda(p["a"]), cuda(sa)), (cuda(p["b"]), cuda(sb)), d, recipe=(1, 1, 128), pack_ue8m0=pack)
    torch.cuda.synchronize()
    o, T = oracle.gemm_nt(p["a"], sa, p["b"], sb, 128, want_abs=True)
    ok, st = check_fp32(d.cpu().numpy(), o, T)
    say("small-n raw block scales", st)
    assert ok.all(), st


def test_ue8m0_code_zero_is_two_to_the_minus_127():
    """UE8M0 is a pure 8-bit exponent, so every code is a power of two (page "02 · DeepGEMM
    技术解析" §3.1): code 0 is 2^-127, the smallest, and the matrix unit applies it as such.
    An FP32 scale of 0.0 passes the page's power-of-two mask and packs to code 0, so its K
    block is scaled by 2^-127 rather than dropped.  Integer payloads make every partial exact;
    large weight scales keep the scaled results out of the FP32 subnormal range."""
    M, N, K = 64, 256, 512
    p = gen.pow2_exact(M, N, K, seed=23)
    sa = p["sa"].copy()
    sa[:8, :] = 0.0              # every block of rows 0..7: code 0
    sa[8:16, 1] = 0.0            # one block of rows 8..15
    sb = (p["sb"] * np.float32(2.0 ** 12)).astype(np.float32)
    say("ue8m0 code 0")
    d = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    dg.fp8_gemm_nt((cuda(p["a"]), cuda(sa)), (cuda(p["b"]), cuda(sb)), d, recipe=(1, 1, 128), pack_ue8m0=True)
    torch.cuda.synchronize()
    words, cnt = oracle.transform_sf(sa, M, 1, True)
    assert cnt == 0                                   # 0.0 passes the power-of-two mask
    sa_dec = oracle.unpack_ue8m0(words, M, K // 128)
    assert (sa_dec[:8] == 2.0 ** -127).all()
    o, T = oracle.gemm_nt(p["a"], sa_dec, p["b"], sb, 128, want_abs=True)
    got = d.cpu().numpy()
    ok, st = check_fp32(got, o, T)
    say("ue8m0 code 0", st)
    assert ok.all(), st
    nz = o[:8] != 0
    assert nz.any() and (got[:8][nz] != 0).all()      # scaled by 2^-127, not dropped
    assert np.array_equal(got.astype(np.float64), o)  # and exactly so


@contextlib.contextmanager
def env_var(name, value):
    old = os.environ.get(name)
    os.environ[name] = str(value)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = old


@pytest.mark.parametrize("bn", [16, 32])
@pytest.mark.parametrize("shape", [(1, 300, 128), (5, 100, 256), (17, 520, 2048), (64, 1000, 1152), (33, 7, 384)])
def test_skinny_decode_shapes(bn, shape):
    """Dense problems with at most 64 rows run the skinny kernel (each workgroup's waves split
    K and add their partial sums at the end): ragged m and n (n below one column block too),
    K from one block up, both column widths, BF16, FP32 and FP32 + C, with sentinels around D."""
    M, N, K = shape
    p = gen.dense(M, N, K, seed=M * 7 + N + K, with_c=True)
    for out, with_c in ((torch.bfloat16, False), (torch.float32, False), (torch.float32, True)):
        say("skinny", shape, bn, out, with_c)
        big = torch.full((M, N + 12), float("nan"), dtype=out, device=DEV)
        d = big[:, :N]
        c = cuda(p["c"]) if with_c else None
        with env_var("DG_SKINNY_BN", bn):
            dg.fp8_gemm_nt((cuda(p["a"]), cuda(p["sa"])), (cuda(p["b"]), cuda(p["sb"])), d, c=c)
        torch.cuda.synchronize()
        st = check_dense(p, d, with_c=with_c, name=f"skinny {shape} {bn}")
        assert torch.isnan(big[:, N:].float()).all()


@pytest.mark.parametrize("G", [64, 66])
def test_k_grouped_many_groups(G):
    """Up to 64 non-empty groups run as one launch over every group's tiles; beyond that, one
    launch per 64 groups.  Groups of one to three K blocks, some empty, C separate."""
    rng = np.random.default_rng(G)
    ks = [int(x) * 128 for x in rng.integers(0, 4, G)]
    ks[0], ks[-1] = 128, 384
    m, n = 96, 260
    nonempty = sum(k > 0 for k in ks)
    p = gen.k_grouped(m, n, ks, seed=G)
    say("k-grouped many groups", G, nonempty)
    c = cuda(p["c"])
    d = torch.full_like(c, float("nan"))
    dg.k_grouped_fp8_gemm_nt_contiguous((cuda(p["a"]), cuda(np.ascontiguousarray(p["sa"].T))),
                                        (cuda(p["b"]), cuda(np.ascontiguousarray(p["sb"].T))), d, ks, c)
    torch.cuda.synchronize()
    o, T = oracle.k_grouped(p["a"], p["sa"], p["b"], p["sb"], ks, p["c"], want_abs=True)
    got = d.cpu().numpy()
    ok, st = check_fp32(got, o, T)
    say("k-grouped many groups", st)
    assert ok.all(), st
    for g, k in enumerate(ks):
        if k == 0:
            assert np.array_equal(got[g], p["c"][g])


def test_k_grouped_single_launch_equals_group_loop():
    """The one-launch K-grouped kernel and one launch per group (same tile, same per-element
    order of MFMAs and promotions) give the same bits."""
    ks = [256, 0, 640, 128, 1024]
    m, n = 516, 516
    p = gen.k_grouped(m, n, ks, seed=77)
    say("k-grouped single vs loop")
    args = ((cuda(p["a"]), cuda(np.ascontiguousarray(p["sa"].T))), (cuda(p["b"]), cuda(np.ascontiguousarray(p["sb"].T))))
    outs = []
    for loop in (False, True):
        d = torch.full_like(cuda(p["c"]), float("nan"))
        with force_tile("256x256"), env_var("DG_KGROUP_LOOP", int(loop)):
            dg.k_grouped_fp8_gemm_nt_contiguous(*args, d, ks, cuda(p["c"]))
        torch.cuda.synchronize()
        outs.append(d.cpu())
    assert torch.equal(outs[0], outs[1])
    o, T = oracle.k_grouped(p["a"], p["sa"], p["b"], p["sb"], ks, p["c"], want_abs=True)
    ok, st = check_fp32(outs[0].numpy(), o, T)
    assert ok.all(), st
