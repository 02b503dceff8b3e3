"""GPU parity of the nn / tn / tt operand layouts (page "第13章 DeepGEMM" §13.3: D = C + A @ B with
the suffix letters giving the transposition of A and B; page "02 · DeepGEMM 技术解析" §5.1: the nn
form of the M-grouped contiguous GEMM) through the C ABI.

An operand stored [K, M] or [K, N] is staged differently from a [M, K] one but feeds the matrix
unit the same bytes in the same registers, so each layout must reproduce the NT result on the same
tile bit for bit; each is also checked against the float64 oracle read through its storage.  The
stored operands carry padding columns (ld > M or N) filled with E4M3 NaN codes: a kernel that read
them into a stored output would fail both checks."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_amd as dg
import oracle
from tests import gen
from tests.test_gpu_parity import DEV, assert_full_size, bf16_bits, cuda, force_tile, say
from tests.tolerance import check_bf16, check_fp32

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


def stored_t(x, pad=16):
    """[R, K] logical operand -> [K, R] stored with row stride align16(R) + pad; the padding
    columns hold NaN codes.  Returns the device view [K, R]."""
    R, K = x.shape
    ld = (R + 15) // 16 * 16 + pad
    buf = np.full((K, ld), NAN_CODE, np.uint8)
    buf[:, :R] = x.T
    return cuda(buf)[:, :R]


def operands(layout, p, pad=16):
    a = cuda(p["a"]) if layout[0] == "n" else stored_t(p["a"], pad)
    b = cuda(p["b"]) if layout[1] == "t" else stored_t(p["b"], pad)
    return a, b


def run(layout, p, out, tile, with_c=False, pack=False, pad=16):
    a, b = operands(layout, p, pad)
    d = torch.full((p["M"], p["N"]), float("nan"), dtype=out, device=DEV)
    c = cuda(p["c"]) if with_c else None
    with force_tile(tile):
        getattr(dg, "fp8_gemm_" + layout)((a, cuda(p["sa"])), (b, cuda(p["sb"])), d, c=c, pack_ue8m0=pack)
    torch.cuda.synchronize()
    return d


def check(p, d, with_c, name=None):
    o, T = oracle.gemm_nt(p["a"], p["sa"], p["b"], p["sb"], 128, c=p["c"] if with_c else None, want_abs=True)
    if d.dtype == torch.bfloat16:
        return check_bf16(bf16_bits(d), o, T, name=name)
    return check_fp32(d.cpu().numpy(), o, T, name=name)


@pytest.mark.parametrize("layout,tile", [(l, t) for l in ("nn", "tn", "tt") for t in ("256x224", "128x192")] +
                         [("nn", "128x256")])
@pytest.mark.parametrize("shape", [(200, 300, 384), (257, 513, 256), (33, 129, 640), (64, 32, 1024), (130, 260, 512)])
def test_layout_equals_nt_bitwise_and_oracle(layout, tile, shape):
    """Ragged m and n on every tile (including fewer rows or columns than one tile), K from
    the two-block minimum up, BF16 and FP32 out (and FP32 + C on the tile that has it).  On
    128x256 (nn), B stored [K, N] takes the row-XOR staging and 8 waves, the NT kernel 4 waves:
    the same partials promoted in the same order, so still the same bits."""
    M, N, K = shape
    p = gen.dense(M, N, K, seed=M * 7 + N + K, with_c=True)
    outs = [(torch.bfloat16, False), (torch.float32, False)] + ([(torch.float32, True)] if tile == "128x192" else [])
    for out, with_c in outs:
        say("layout", layout, shape, tile, out, "C" if with_c else "")
        d_nt = run("nt", p, out, tile, with_c)
        d = run(layout, p, out, tile, with_c)
        assert torch.equal(d.view(torch.int16) if out == torch.bfloat16 else d.view(torch.int32),
                           d_nt.view(torch.int16) if out == torch.bfloat16 else d_nt.view(torch.int32)), \
            (layout, shape, tile, out)
        ok, st = check(p, d, with_c)
        say("layout", layout, st)
        assert ok.all(), st


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("tile", ["256x224", "128x192"])
def test_layout_ue8m0_scales(layout, tile):
    """Packed UE8M0 scales (applied by the matrix unit) with operands stored [K, x]."""
    M, N, K = 300, 450, 768
    p = gen.pow2_exact(M, N, K, seed=3)
    p["sb"] = oracle.expand_scales_b(p["sb"], N, 128).astype(np.float32)   # one scale per weight row
    for out in (torch.bfloat16, torch.float32):
        say("layout ue8m0", layout, tile, out)
        a, b = operands(layout, p)
        d = torch.full((M, N), float("nan"), dtype=out, device=DEV)
        with force_tile(tile):
            getattr(dg, "fp8_gemm_" + layout)((a, cuda(p["sa"])), (b, cuda(p["sb"])), d, recipe=(1, 1, 128),
                                              pack_ue8m0=True)
        torch.cuda.synchronize()
        o = oracle.gemm_nt(p["a"], p["sa"], p["b"], p["sb"], 1)
        if out == torch.float32:
            assert np.array_equal(d.cpu().numpy().astype(np.float64), o)     # every partial is exact
        else:
            assert np.array_equal(bf16_bits(d), oracle.bf16_rne(o))


def test_layout_planner_tiles_and_c_aliasing():
    """The planner's own tile choice (no forced tile) for a small and a large problem, and C
    accumulated in place in D with A stored [K, M]."""
    for (M, N, K) in [(16, 48, 256), (1000, 1500, 512)]:
        p = gen.dense(M, N, K, seed=M + 1, with_c=True)
        for layout in ("nn", "tn", "tt"):
            say("layout planner", layout, M, N, K)
            d = run(layout, p, torch.bfloat16, None)
            ok, st = check(p, d, False)
            assert ok.all(), (layout, st)
    p = gen.dense(192, 320, 512, seed=9, with_c=True)
    a, b = operands("tt", p)
    d = cuda(p["c"]).clone()
    say("layout tt C aliased")
    dg.fp8_gemm_tt((a, cuda(p["sa"])), (b, cuda(p["sb"])), d, c=d)
    torch.cuda.synchronize()
    ok, st = check(p, d, True)
    assert ok.all(), st


@pytest.mark.parametrize("layout", ["tn", "nn"])
def test_layout_full_size_sampled_rows(layout):
    """tn (both operands stored K-outermost, the weight-gradient storage) and nn (B stored
    [K, N]) at the dense benchmark size, M = 4096, N = 7168, K = 2048, BF16 out, in the
    planner's launch configuration (nn: the 256-wide tile); rows are independent, so 384
    sampled rows (first and last included) are checked."""
    p = gen.dense(4096, 7168, 2048, seed=0)
    say("layout full size", layout)
    d = run(layout, p, torch.bfloat16, None, pad=0)
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(4).choice(4096, 382, replace=False)]))
    o, T = oracle.gemm_nt(p["a"][rows], p["sa"][rows], p["b"], p["sb"], 128, want_abs=True)
    ok, st = check_bf16(bf16_bits(d)[rows], o, T, name=f"{layout} 4096x7168x2048 ({len(rows)} rows) bf16")
    say("layout full size", layout, st)
    assert ok.all(), st
    assert_full_size(st, f"{layout} dense")


def test_m_grouped_nn_contiguous_full_size_equals_nt():
    """The contiguous workload the benchmark times (32 groups, 4096 x 7168 weights) with the
    weights stored [K, N], in the planner's launch configuration: every output equals the NT
    form's bit for bit (the NT form is checked against the oracle at this size elsewhere)."""
    p = gen.config4()
    say("m-grouped nn full size", p["M"], p["N"], p["K"])
    a, sa, lay = cuda(p["a"]), cuda(p["sa"]), cuda(p["layout"])
    outs = []
    for form, b in (("nt", cuda(p["b"])), ("nn", cuda(np.ascontiguousarray(np.swapaxes(p["b"], 1, 2))))):
        d = torch.full((p["M"], p["N"]), float("nan"), dtype=torch.bfloat16, device=DEV)
        getattr(dg, f"m_grouped_fp8_gemm_{form}_contiguous")((a, sa), (b, cuda(p["sb"])), d, lay)
        torch.cuda.synchronize()
        outs.append(d.view(torch.int16).cpu())
        del b
    assert torch.equal(outs[0], outs[1])


def test_m_grouped_nn_contiguous_ragged():
    """Contiguous groups with each group's weights stored [K, N]: equal to the NT form bit for
    bit on the same tile, and to the oracle; padding rows, a skipped block, m_total cut inside
    the last block, ragged n, NaN sentinels on rows that produce no output."""
    G, N, K = 4, 300, 512
    p = gen.grouped_contiguous(G, N, K, seed=31, m_units=(1, 3))
    starts = np.concatenate([[0], np.cumsum(p["sizes"])])
    layout = p["layout"].copy()
    layout[starts[2] - 40:starts[2]] = -1
    if p["sizes"][2] > 128:
        layout[starts[2]:starts[2] + 128] = -1
    M = p["M"] - 30
    a, sa, layout = p["a"][:M], p["sa"][:M], layout[:M]
    ld = (N + 15) // 16 * 16 + 16
    bt = np.full((G, K, ld), NAN_CODE, np.uint8)
    bt[:, :, :N] = np.swapaxes(p["b"], 1, 2)
    b_nn = cuda(bt)[:, :, :N]
    for tile in ("128x256", "128x224"):
        for out in (torch.bfloat16, torch.float32):
            say("m-grouped nn", tile, out, p["sizes"].tolist(), M)
            ds = []
            for form, b in (("nt", cuda(p["b"])), ("nn", b_nn)):
                d = torch.full((M, N), float("nan"), dtype=out, device=DEV)
                with force_tile(tile):
                    getattr(dg, f"m_grouped_fp8_gemm_{form}_contiguous")((cuda(a), cuda(sa)), (b, cuda(p["sb"])), d,
                                                                          cuda(layout))
                torch.cuda.synchronize()
                ds.append(d)
            assert torch.equal(ds[0].float().isnan(), ds[1].float().isnan())
            assert torch.equal(torch.nan_to_num(ds[0].float()), torch.nan_to_num(ds[1].float()))
            o, T = oracle.grouped_contiguous_nn(a, sa, np.swapaxes(p["b"], 1, 2), p["sb"], layout, want_abs=True)
            live = ~np.isnan(o)
            got = ds[1]
            if out == torch.bfloat16:
                ok, st = check_bf16(bf16_bits(got)[live], o[live], T[live])
            else:
                ok, st = check_fp32(got.cpu().numpy()[live], o[live], T[live])
            say("m-grouped nn", st)
            assert ok.all(), st
            assert np.isnan(got.float().cpu().numpy()[~live]).all()


def test_m_grouped_nn_contiguous_ue8m0():
    """Contiguous groups with weights stored [K, N] and packed UE8M0 scales (power-of-two scales,
    one per weight row), on both nn tiles: bit for bit equal to the NT form on the same tile, and
    to the oracle evaluated with the same scales; a skipped block and rows past m_total."""
    G, N, K = 4, 300, 512
    p = gen.grouped_contiguous(G, N, K, seed=41, m_units=(1, 3))
    pow2 = lambda x: np.exp2(np.ceil(np.log2(x))).astype(np.float32)   # scales rounded up to 2^e
    sa = pow2(p["sa"])
    sb = np.stack([oracle.expand_scales_b(pow2(p["sb"][g]), N, 128) for g in range(G)]).astype(np.float32)
    starts = np.concatenate([[0], np.cumsum(p["sizes"])])
    layout = p["layout"].copy()
    if p["sizes"][1] > 128:
        layout[starts[1]:starts[1] + 128] = -1
    M = p["M"] - 20
    a, sa, layout = p["a"][:M], sa[:M], layout[:M]
    ld = (N + 15) // 16 * 16                             # rows of [K, N] padded to 16 bytes
    bt = np.full((G, K, ld), NAN_CODE, np.uint8)
    bt[:, :, :N] = np.swapaxes(p["b"], 1, 2)
    b_nn = cuda(bt)[:, :, :N]
    o, T = oracle.grouped_contiguous(a, sa, p["b"], sb, layout, gran_n=1, want_abs=True)
    live = ~np.isnan(o)
    for tile in ("128x256", "128x224"):
        say("m-grouped nn ue8m0", tile, p["sizes"].tolist(), M)
        ds = []
        for form, b in (("nt", cuda(p["b"])), ("nn", b_nn)):
            d = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
            with force_tile(tile):
                getattr(dg, f"m_grouped_fp8_gemm_{form}_contiguous")((cuda(a), cuda(sa)), (b, cuda(sb)), d,
                                                                      cuda(layout), recipe=(1, 1, 128), pack_ue8m0=True)
            torch.cuda.synchronize()
            ds.append(d.view(torch.int16).cpu())
        assert torch.equal(ds[0], ds[1]), tile
        bits = ds[1].numpy().view(np.uint16)
        ok, st = check_bf16(bits[live], o[live], T[live])
        say("m-grouped nn ue8m0", st)
        assert ok.all(), st
        assert (bits[~live] == np.uint16(0x7FC0)).all()      # rows that produce no output keep the NaN


@pytest.mark.parametrize("tile", ["256x224", "128x192"])
@pytest.mark.parametrize("shape", [(200, 300, 384), (33, 129, 640), (257, 64, 256)])
def test_fp8_fp4_tt_equals_nt_bitwise_and_oracle(tile, shape):
    """FP8 x FP4 with the activations stored [K, M] next to K-packed FP4 weights."""
    M, N, K = shape
    p = gen.fp8_fp4(M, N, K, seed=M + N, with_c=True)
    outs = [(torch.bfloat16, False), (torch.float32, False)] + ([(torch.float32, True)] if tile == "128x192" else [])
    for out, with_c in outs:
        say("fp8 x fp4 tt", shape, tile, out, with_c)
        res = []
        for form, a in (("nt", cuda(p["a"])), ("tt", stored_t(p["a"]))):
            d = torch.full((M, N), float("nan"), dtype=out, device=DEV)
            with force_tile(tile):
                getattr(dg, "fp8_fp4_gemm_" + form)((a, cuda(p["sa"])), (cuda(p["b"]), cuda(p["sb"])), d,
                                                    c=cuda(p["c"]) if with_c else None)
            torch.cuda.synchronize()
            res.append(d)
        assert torch.equal(res[0].view(torch.int16) if out == torch.bfloat16 else res[0].view(torch.int32),
                           res[1].view(torch.int16) if out == torch.bfloat16 else res[1].view(torch.int32))
        o, T = oracle.gemm_fp8_fp4_tt(np.ascontiguousarray(p["a"].T), p["sa"], p["b"], p["sb"],
                                      c=p["c"] if with_c else None, want_abs=True)
        if out == torch.bfloat16:
            ok, st = check_bf16(bf16_bits(res[1]), o, T)
        else:
            ok, st = check_fp32(res[1].cpu().numpy(), o, T)
        say("fp8 x fp4 tt", st)
        assert ok.all(), st


@pytest.mark.parametrize("layout,tile", [("nt", "256x224"), ("nt", "128x192"), ("tt", "256x224"), ("nn", "256x224"),
                                         ("tn", "128x192")])
def test_largest_leading_dimension(layout, tile):
    """Operands at the largest leading dimension the boundary accepts, every other byte of their
    buffers a NaN code: a K-major operand with ld = 2^23 - 16 bytes (the byte range of a
    256-row tile is then 2^31 - 4096, the most a signed 32-bit range holds) and an MN-major one
    with k * ld just below 2^31 (k = 256).  Checked element by element against the oracle."""
    M, N, K = 256, 224, 256
    LD = (1 << 23) - 16
    p = gen.dense(M, N, K, seed=23)

    def place(x, mn_major):
        src = cuda(np.ascontiguousarray(x.T) if mn_major else x)
        buf = torch.full((src.shape[0], LD), NAN_CODE, dtype=torch.uint8, device=DEV)
        buf[:, :src.shape[1]] = src
        return buf[:, :src.shape[1]]

    say("largest ld", layout, tile, LD)
    a = place(p["a"], layout[0] == "t")
    b = place(p["b"], layout[1] == "n")
    d = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    with force_tile(tile):
        getattr(dg, "fp8_gemm_" + layout)((a, cuda(p["sa"])), (b, cuda(p["sb"])), d)
    torch.cuda.synchronize()
    del a, b
    o, T = oracle.gemm_nt(p["a"], p["sa"], p["b"], p["sb"], 128, want_abs=True)
    ok, st = check_bf16(bf16_bits(d), o, T)
    say("largest ld", layout, tile, st)
    assert ok.all(), st


def _k_grouped_operands(p, layout, pad=16):
    if layout == "nt":
        return cuda(p["a"]), cuda(p["b"])
    return stored_t(p["a"], pad), stored_t(p["b"], pad)


@pytest.mark.parametrize("m,n,ks,tile", [(260, 196, [256, 0, 384, 128, 512], None), (64, 520, [128], None),
                                         (4, 4, [0, 128, 0], None), (516, 388, [1024, 128, 0, 640], None),
                                         (516, 388, [1024, 128, 0, 640], "256x224"),
                                         (516, 388, [1024, 128, 0, 640], "256x256"),
                                         (300, 452, [384, 256, 0, 128], "256x224"),
                                         (300, 452, [384, 256, 0, 128], "256x256"),
                                         (300, 452, [384, 256, 0, 128], "128x224")])
def test_k_grouped_tn_equals_nt_bitwise_and_oracle(m, n, ks, tile):
    """K-grouped GEMM with both operands stored K-outermost ([sum K, m] and [sum K, n], the
    token-major storage of the weight-gradient operands): the NT result bit for bit, and the
    oracle read through the storage; empty groups give C, C accumulated in place.  Forced on
    ragged shapes to 256x256 (both operands staged row-XOR), 256x224 (A row-XOR, B in strips)
    and 128x224 (both in strips)."""
    p = gen.k_grouped(m, n, ks, seed=m + n + 3 * len(ks))
    sfa, sfb = cuda(np.ascontiguousarray(p["sa"].T)), cuda(np.ascontiguousarray(p["sb"].T))
    outs = {}
    for layout in ("nt", "tn"):
        say("k-grouped", layout, m, n, ks, tile)
        a, b = _k_grouped_operands(p, layout)
        d = cuda(p["c"]).clone()
        with force_tile(tile if layout == "tn" else None):
            getattr(dg, f"k_grouped_fp8_gemm_{layout}_contiguous")((a, sfa), (b, sfb), d, ks, d)
        torch.cuda.synchronize()
        outs[layout] = d.cpu()
    assert torch.equal(outs["nt"].view(torch.int32), outs["tn"].view(torch.int32))
    o, T = oracle.k_grouped_tn(np.ascontiguousarray(p["a"].T), p["sa"], np.ascontiguousarray(p["b"].T), p["sb"],
                               ks, p["c"], want_abs=True)
    ok, st = check_fp32(outs["tn"].numpy(), o, T)
    say("k-grouped tn", st)
    assert ok.all(), st
    for g, k in enumerate(ks):
        if k == 0:
            assert np.array_equal(outs["tn"].numpy()[g], p["c"][g])


def test_k_grouped_tn_full_size_equals_nt():
    """The K-grouped weight-gradient workload at the size the benchmark times (m = 7168,
    n = 2048, eight groups, K = 16384 in all), with token-major operands on the tile the planner
    picks: the whole output bit for bit equal to the NT form's (whose full-size result is
    checked against the oracle on sampled outputs), C accumulated in place."""
    ks = [1792, 2304, 2048, 1536, 2560, 2048, 1920, 2176]
    m, n = 7168, 2048
    p = gen.k_grouped(m, n, ks, seed=9)
    sfa, sfb = cuda(np.ascontiguousarray(p["sa"].T)), cuda(np.ascontiguousarray(p["sb"].T))
    outs = {}
    for layout in ("nt", "tn"):
        say("k-grouped full size", layout)
        a, b = _k_grouped_operands(p, layout, pad=0)
        d = cuda(p["c"])
        getattr(dg, f"k_grouped_fp8_gemm_{layout}_contiguous")((a, sfa), (b, sfb), d, ks, d)
        torch.cuda.synchronize()
        outs[layout] = d
        del a, b
    assert torch.equal(outs["nt"].view(torch.int32), outs["tn"].view(torch.int32))


def test_k_grouped_tn_more_than_64_groups():
    """70 groups (some empty) with token-major operands: two launches of up to 64 groups, each
    group into its own output, against the oracle; C read separately."""
    rng = np.random.default_rng(70)
    ks = [int(x) * 128 for x in rng.integers(0, 3, 70)]
    ks[0], ks[-1] = 256, 128
    m, n = 96, 132
    p = gen.k_grouped(m, n, ks, seed=70)
    say("k-grouped tn 70 groups", sum(k > 0 for k in ks))
    a, b = _k_grouped_operands(p, "tn", pad=0)
    c = cuda(p["c"])
    d = torch.full_like(c, float("nan"))
    dg.k_grouped_fp8_gemm_tn_contiguous((a, cuda(np.ascontiguousarray(p["sa"].T))),
                                        (b, cuda(np.ascontiguousarray(p["sb"].T))), d, ks, c)
    torch.cuda.synchronize()
    o, T = oracle.k_grouped(p["a"], p["sa"], p["b"], p["sb"], ks, p["c"], want_abs=True)
    ok, st = check_fp32(d.cpu().numpy(), o, T)
    say("k-grouped tn 70 groups", st)
    assert ok.all(), st
