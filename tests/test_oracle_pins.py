"""Pins for the float64 oracle: each oracle function is checked against
something other than itself -- closed forms, worked examples printed on the
pages (tests/golden/), exact rational brute force on tiny inputs, library
routines on special cases, and invariants.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs, layout, gemm
from tests import gen
from tests.tolerance import check_bf16, check_fp32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


# ---------------------------------------------------------------- E4M3 decode
def test_e4m3_hand_values():
    t = codecs.e4m3_decode_table()
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2


def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = codecs.e4m3_decode_table()
    same = (t == ref) | (np.isnan(t) & np.isnan(ref))
    assert same.all()


# ---------------------------------------------------------------- UE8M0
@pytest.mark.parametrize("fixture", ["ue8m0_examples.txt", "ue8m0_closed_form.txt"])
def test_ue8m0_examples(fixture):
    for val, code, dec, bad in _rows(fixture):
        x = np.float32(float(val))
        c = codecs.ue8m0_encode(np.array([x]))[0]
        assert int(c) == int(code), (val, c)
        assert codecs.ue8m0_decode(np.array([c]))[0] == float(dec)
        assert bool(codecs.pow2_violation(np.array([x]))[0]) == bool(int(bad))


def test_ue8m0_special_codes():
    assert np.isnan(codecs.ue8m0_decode(np.array([255], np.uint8))[0])
    # the format is a bare exponent: code 0 is the smallest power of two, not zero
    assert codecs.ue8m0_decode(np.array([0], np.uint8))[0] == 2.0 ** -127
    assert codecs.ue8m0_decode(np.array([1], np.uint8))[0] == 2.0 ** -126
    # every code 1..254 decodes to 2^(code - 127)
    c = np.arange(1, 255, dtype=np.uint8)
    assert (codecs.ue8m0_decode(c) == np.ldexp(1.0, c.astype(np.int32) - 127)).all()


# ---------------------------------------------------------------- BF16 RNE
def _bf16_exact(x):
    """Correct RNE of a float64 to BF16 by exact rationals (brute force)."""
    if x == 0:
        return 0x8000 if np.signbit(x) else 0
    sign = 0x8000 if x < 0 else 0
    fx = abs(Fraction(x))
    e = -126
    while fx >= Fraction(2) ** (e + 1):
        e += 1
    while e > -126 and fx < Fraction(2) ** e:
        e -= 1
    sp = Fraction(2) ** (e - 7)
    q = fx / sp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * sp
    if val > Fraction(2) ** 127 * (2 - Fraction(1, 128)):
        return sign | 0x7F80
    bits = int(np.float32(float(val)).view(np.uint32)) >> 16
    return sign | bits


def test_bf16_constructed_ties():
    cases = [(1 + 2.0 ** -8, 0x3F80), (1 + 3 * 2.0 ** -8, 0x3F82), (1 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),
             (-(1 + 2.0 ** -8), 0xBF80), (0.0, 0x0000), (-0.0, 0x8000),
             ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),       # tie at the top rounds up to infinity
             ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),
             (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -135, 0x0001), (3 * 2.0 ** -134, 0x0002), (2.0 ** -134 + 2.0 ** -140, 0x0001)]
    for x, bits in cases:
        assert int(codecs.bf16_rne(np.array([x]))[0]) == bits, (x, hex(bits))


def test_bf16_random_vs_exact_rationals():
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(1500) * np.exp2(rng.integers(-140, 130, 1500)),
        rng.standard_normal(300),
        # exact ties between neighbouring BF16 values
        (rng.integers(256, 512, 200) * 2 + 1) * np.exp2(rng.integers(-20, 20, 200) - 9.0),
    ])
    got = codecs.bf16_rne(xs)
    for x, g in zip(xs, got):
        assert int(g) == _bf16_exact(float(x)), x


def test_bf16_matches_torch_on_float32_inputs():
    # torch's float32 -> bfloat16 cast is a single RNE step; on float32 inputs it must agree
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(100000) * np.exp2(rng.integers(-60, 60, 100000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (codecs.bf16_rne(x32.astype(np.float64)) == ref).all()


# ---------------------------------------------------------------- layout transform
def test_transform_hand_example_fp32():
    # mn = 6 rows, sf_k = 5 K-blocks: align4(6) = 8, element (r, kb) lands at kb*8 + r
    sf = np.arange(30, dtype=np.float32).reshape(6, 5) + 1      # value = 5r + kb + 1
    out, _ = layout.transform_sf(sf, 6, 1, False)
    assert out.shape == (5, 8)
    flat = out.reshape(-1)
    assert flat[0] == 1 and flat[1] == 6 and flat[5] == 26       # kb=0: rows 0, 1, 5
    assert flat[8] == 2 and flat[8 * 4 + 5] == 30               # kb=1 row 0; kb=4 row 5
    assert (out[:, 6:] == 0).all()                              # padding rows are 0


def test_transform_hand_example_packed():
    # exponents chosen so that the codes are 100 + 10r + kb
    codes = np.array([[100 + 10 * r + kb for kb in range(5)] for r in range(6)], dtype=np.uint32)
    sf = (codes << np.uint32(23)).view(np.float32)
    out, cnt = layout.transform_sf(sf, 6, 1, True)
    assert cnt == 0 and out.shape == (2, 8) and out.dtype == np.int32
    w = out.view(np.uint32)
    # word (r=2, q=0) = codes of K-blocks 0..3 of row 2, little-endian: 120,121,122,123
    assert w[0, 2] == 120 | 121 << 8 | 122 << 16 | 123 << 24
    # word (r=2, q=1): only K-block 4 exists -> byte 0 = 124, bytes 1..3 = 0
    assert w[1, 2] == 124
    assert (w[:, 6:] == 0).all()


def test_transform_broadcast_gran128_and_count():
    sf = np.array([[0.75, 1.0], [3.0, 0.5]], dtype=np.float32)   # two 128-row blocks, sf_k = 2
    out, cnt = layout.transform_sf(sf, 200, 128, True)
    assert cnt == 2                                             # 0.75 and 3.0 are not powers of two
    w = out.view(np.uint32)
    assert out.shape == (1, 200)
    assert w[0, 0] == 126 | 127 << 8 and w[0, 127] == 126 | 127 << 8
    assert w[0, 128] == 128 | 126 << 8 and w[0, 199] == 128 | 126 << 8
    fp, _ = layout.transform_sf(sf, 200, 128, False)
    assert fp.shape == (2, 200) and fp[0, 127] == np.float32(0.75) and fp[1, 128] == np.float32(0.5)


def test_unpack_roundtrip():
    rng = np.random.default_rng(3)
    sf = np.exp2(rng.integers(-20, 20, size=(3, 37, 7))).astype(np.float32)
    out, cnt = layout.transform_sf(sf, 37, 1, True)
    assert cnt == 0
    back = layout.unpack_ue8m0(out, 37, 7)
    assert (back == sf).all()


# ---------------------------------------------------------------- GEMM core vs brute force
def _brute(a, sa, b, sb, gran_n, c=None):
    """Exact rational value of the definition, and sum |A'B'|."""
    M, K = a.shape
    N = b.shape[0]
    t = codecs.e4m3_decode_table()
    D = np.empty((M, N))
    T = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            tot = Fraction(0)
            for k in range(K):
                s = Fraction(float(sa[i, k // 128])) * Fraction(float(sb[j // gran_n, k // 128]))
                p = Fraction(float(t[a[i, k]])) * Fraction(float(t[b[j, k]])) * s
                acc += p
                tot += abs(p)
            if c is not None:
                acc += Fraction(float(c[i, j]))
            D[i, j] = float(acc)
            T[i, j] = float(tot)
    return D, T


def _random_tiny(rng, M, N, K, gran_n):
    codes = np.concatenate([np.arange(0, 0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)  # no NaN
    a = rng.choice(codes, size=(M, K))
    b = rng.choice(codes, size=(N, K))
    sf_k = (K + 127) // 128
    sa = (rng.random((M, sf_k)) * 3 + 1e-3).astype(np.float32)
    nb = (N + gran_n - 1) // gran_n
    sb = (rng.random((nb, sf_k)) * 3 + 1e-3).astype(np.float32)
    return a, sa, b, sb


@pytest.mark.parametrize("K", [128, 256, 384, 200])
@pytest.mark.parametrize("gran_n", [128, 1])
def test_gemm_vs_brute_force(K, gran_n):
    rng = np.random.default_rng(K + gran_n)
    M, N = 5, 7
    a, sa, b, sb = _random_tiny(rng, M, N, K, gran_n)
    c = rng.standard_normal((M, N)).astype(np.float32)
    D, T = gemm.gemm_nt(a, sa, b, sb, gran_n, c=c, want_abs=True)
    Dx, Tx = _brute(a, sa, b, sb, gran_n, c)
    assert np.all(np.abs(D - Dx) <= 2.0 ** -48 * (Tx + np.abs(c)))
    assert np.allclose(T, Tx, rtol=1e-14, atol=0)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Dp, Tp = gemm.gemm_nt_points(a, sa, b, sb, ii.ravel(), jj.ravel(), gran_n, c=c)
    assert np.all(np.abs(Dp - Dx.ravel()) <= 2.0 ** -48 * (Tx.ravel() + np.abs(c).ravel()))


def test_gemm_1d2d_block_boundary_brute_force():
    # N = 300 crosses two 128-column weight-scale boundaries; check columns around them
    rng = np.random.default_rng(7)
    a, sa, b, sb = _random_tiny(rng, 3, 300, 256, 128)
    D = gemm.gemm_nt(a, sa, b, sb, 128)
    for j in [0, 127, 128, 255, 256, 299]:
        Dj, _ = _brute(a, sa, b[j:j + 1], sb[j // 128:j // 128 + 1], 128)
        assert np.all(np.abs(D[:, j] - Dj[:, 0]) <= 1e-12 * np.abs(Dj[:, 0]).max())


def test_all_ones_scales_equal_plain_fp8_matmul():
    d = gen.tiny_dense(seed=5)
    sa = np.ones_like(d["sa"])
    sb = np.ones_like(d["sb"])
    D = gemm.gemm_nt(d["a"], sa, d["b"], sb, 128)
    ref = codecs.e4m3_decode(d["a"]) @ codecs.e4m3_decode(d["b"]).T
    assert np.array_equal(D, ref)     # bitwise: every block partial and their sum are exact


def test_dequantize_then_matmul_formulation():
    # the dequantize-then-matmul statement: (A * S_A) @ (B * S_B)^T + C with the scales expanded
    d = gen.dense(64, 300, 384, seed=6, with_c=True)
    A = codecs.e4m3_decode(d["a"]) * np.repeat(d["sa"].astype(np.float64), 128, axis=1)[:, :384]
    sbe = gemm.expand_scales_b(d["sb"], 300, 128)
    B = codecs.e4m3_decode(d["b"]) * np.repeat(sbe, 128, axis=1)[:, :384]
    ref = A @ B.T + d["c"]
    D, T = gemm.gemm_nt(d["a"], d["sa"], d["b"], d["sb"], 128, c=d["c"], want_abs=True)
    assert np.all(np.abs(D - ref) <= 1e-13 * (T + np.abs(d["c"])))


def test_scale_linearity_exact_on_pow2_inputs():
    d = gen.pow2_exact(16, 40, 512, seed=8)
    D0 = gemm.gemm_nt(d["a"], d["sa"], d["b"], d["sb"], 128)
    sa2 = d["sa"].copy()
    sa2[:, 2] *= 8
    D1 = gemm.gemm_nt(d["a"], sa2, d["b"], d["sb"], 128)
    A = codecs.e4m3_decode(d["a"])[:, 256:384]
    B = codecs.e4m3_decode(d["b"])[:, 256:384]
    contrib = (d["sa"][:, 2:3].astype(np.float64) * d["sb"][0, 2]) * (A @ B.T)
    assert np.array_equal(D1 - D0, 7 * contrib)


def test_grouped_contiguous_vs_brute_force():
    rng = np.random.default_rng(9)
    G, N, K = 3, 6, 256
    rows = np.array([0, 0, 2, 2, 2, -1, 1, 1], dtype=np.int32)   # a padding row included
    M = len(rows)
    a, sa, _, _ = _random_tiny(rng, M, 1, K, 128)
    b = np.stack([_random_tiny(rng, 1, N, K, 128)[2] for _ in range(G)])
    sb = np.stack([_random_tiny(rng, 1, N, K, 128)[3] for _ in range(G)])
    D = gemm.grouped_contiguous(a, sa, b, sb, rows)
    for i, g in enumerate(rows):
        if g < 0:
            assert np.isnan(D[i]).all()
            continue
        Dx, _ = _brute(a[i:i + 1], sa[i:i + 1], b[g], sb[g], 128)
        assert np.allclose(D[i], Dx[0], rtol=1e-13, atol=0)


def test_grouped_masked_vs_brute_force():
    rng = np.random.default_rng(10)
    G, Mmax, N, K = 3, 4, 5, 128
    a = np.stack([_random_tiny(rng, Mmax, 1, K, 128)[0] for _ in range(G)])
    sa = np.stack([_random_tiny(rng, Mmax, 1, K, 128)[1] for _ in range(G)])
    b = np.stack([_random_tiny(rng, 1, N, K, 128)[2] for _ in range(G)])
    sb = np.stack([_random_tiny(rng, 1, N, K, 128)[3] for _ in range(G)])
    masked = np.array([2, 0, 9])        # 9 is clamped to M_max
    D = gemm.grouped_masked(a, sa, b, sb, masked)
    assert np.isnan(D[0, 2:]).all() and np.isnan(D[1]).all() and not np.isnan(D[2]).any()
    for g, m in [(0, 2), (2, 4)]:
        Dx, _ = _brute(a[g, :m], sa[g, :m], b[g], sb[g], 128)
        assert np.allclose(D[g, :m], Dx, rtol=1e-13, atol=0)


def test_per_row_weight_scales_equal_broadcast_block_scales():
    # 1d1d per-row weight scales that repeat the 128x128 block value give the 1d2d result
    d = gen.dense(8, 260, 256, seed=11)
    per_row = gemm.expand_scales_b(d["sb"], 260, 128)
    D2 = gemm.gemm_nt(d["a"], d["sa"], d["b"], d["sb"], 128)
    D1 = gemm.gemm_nt(d["a"], d["sa"], d["b"], per_row, 1)
    assert np.array_equal(D1, D2)


# ---------------------------------------------------------------- the tolerance checks have teeth
def test_tolerance_catches_planted_mistakes():
    d = gen.dense(32, 256, 512, seed=12, with_c=True)
    D, T = gemm.gemm_nt(d["a"], d["sa"], d["b"], d["sb"], 128, c=d["c"], want_abs=True)
    ok, _ = check_fp32(D.astype(np.float32), D, T)
    assert ok.all()
    # a dropped K block
    sa_drop = d["sa"].copy()
    sa_drop[:, 1] = 0
    bad = gemm.gemm_nt(d["a"], sa_drop, d["b"], d["sb"], 128, c=d["c"])
    assert not check_fp32(bad, D, T)[0].all()
    # the wrong weight-scale block for the second half of the columns
    sb_wrong = d["sb"].copy()
    sb_wrong[1] = sb_wrong[0]
    bad = gemm.gemm_nt(d["a"], d["sa"], d["b"], sb_wrong, 128, c=d["c"])
    assert not check_fp32(bad, D, T)[0].all()
    # a missing C term
    bad = gemm.gemm_nt(d["a"], d["sa"], d["b"], d["sb"], 128)
    assert not check_fp32(bad, D, T)[0].all()
    # BF16: correct rounding passes, a one-row shift fails
    bits = oracle.bf16_rne(D)
    assert check_bf16(bits, D, T)[0].all()
    assert not check_bf16(np.roll(bits, 1, axis=0), D, T)[0].all()


def test_tolerance_gates_are_tight():
    """The gates sit at the measured FP8-MFMA ceiling, not far above it: an FP32 error of
    2^-12 * T passes, 2^-11 * T fails; a BF16 result two or three ulps off where |o| is not
    small next to T fails; so does a flood of elements that pass only as cancellations."""
    from tests.tolerance import bf16_ordered, CANCEL_RATIO
    d = gen.dense(64, 256, 512, seed=13)
    D, T = gemm.gemm_nt(d["a"], d["sa"], d["b"], d["sb"], 128, want_abs=True)
    sign = np.where(D >= 0, 1.0, -1.0)
    assert check_fp32(D + sign * 2.0 ** -12 * T, D, T)[0].all()
    ok, st = check_fp32(D + sign * 2.0 ** -11 * T, D, T)
    assert not ok.any() and st["within_1e5"] == 0.0
    bits = oracle.bf16_rne(D)
    big = np.abs(D) > CANCEL_RATIO * T
    assert big.mean() > 0.5
    for k in (2, 3):
        moved = (bf16_ordered(bits) + k).astype(np.int64)
        # back from the ordered image to bit patterns (moving away from zero keeps the sign)
        shifted = np.where(moved < 0, ((-moved) | 0x8000), moved).astype(np.uint16)
        ok, _ = check_bf16(shifted, D, T)
        assert not ok[big & (D > 0)].any(), k
    # elements that pass only as cancellations: within the cap they pass, above it they fail
    tiny = np.zeros_like(D)
    Tc = np.full_like(D, 1.0)
    off = oracle.bf16_rne(np.full_like(D, 2.0 ** -14))     # |d - o| = 2^-14 <= EPS_MMA * T
    ok, st = check_bf16(off, tiny, Tc)
    assert st["cancellation_only"] == D.size and not ok.any()
    ok, st = check_bf16(np.where(np.arange(D.size).reshape(D.shape) == 0, off, oracle.bf16_rne(tiny)), tiny, Tc)
    assert st["cancellation_only"] == 1 and ok.all()


# ---------------------------------------------------------------- the per-token-group cast
def test_e4m3_encode_hand_values():
    from oracle import quant
    vals = [1.0625, 1.1875, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, -448.0, -0.0, 0.0, 0.5, -1.5]
    want = [0x38, 0x3A, 0x01, 0x00, 0x02, 0x7E, 0xFE, 0x80, 0x00, 0x30, 0xBC]
    assert quant.e4m3_encode_rne(vals).tolist() == want


def test_e4m3_encode_inverts_decode():
    from oracle import quant
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(quant.e4m3_encode_rne(codecs.e4m3_decode(codes)), codes)


def test_e4m3_encode_matches_torch_including_ties():
    # torch's float8_e4m3fn cast rounds to nearest even: a library routine on the same values,
    # here on random values and on every midpoint between neighbouring finite values
    from oracle import quant
    rng = np.random.default_rng(31)
    pos = np.sort(codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01, mids, -mids])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quant.e4m3_encode_rne(x), ref)


def test_per_token_group_cast_closed_forms():
    from oracle import quant
    rng = np.random.default_rng(32)
    # a group whose amax is 448 * 2^e has the scale 2^e exactly, and E4M3 values times 2^e
    # come back as the same codes
    codes = rng.integers(0, 0x7E, size=(3, 256)).astype(np.uint8)
    codes[:, 0] = 0x7E                                   # amax 448 in both groups
    codes[:, 128] = 0x7E
    sign = rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    codes = codes | sign
    e = np.array([[-3, 2], [0, -7], [5, 0]])
    x = codecs.e4m3_decode(codes) * np.repeat(2.0 ** e, 128, axis=1)
    q, s = quant.per_token_group_cast(x.astype(np.float32))
    assert np.array_equal(s, (2.0 ** e).astype(np.float32))
    assert np.array_equal(q, codes)
    # an all-zero group: scale 1, codes 0
    q, s = quant.per_token_group_cast(np.zeros((2, 128), np.float32))
    assert np.array_equal(s, np.ones((2, 1), np.float32)) and not q.any()
    # any input: the dequantized value is within half an E4M3 step of x (relative to the scale)
    x = (rng.standard_normal((4, 512)) * np.exp(rng.uniform(-8, 8, (4, 1)))).astype(np.float32)
    q, s = quant.per_token_group_cast(x)
    deq = codecs.e4m3_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    y = np.abs(x.astype(np.float64) / np.repeat(s.astype(np.float64), 128, axis=1))
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
    assert np.all(np.abs(deq - x) <= (step / 2 + 1e-6 * y) * np.repeat(s.astype(np.float64), 128, axis=1))
    assert np.all(codecs.e4m3_decode(q).max(axis=1) <= 448)


def test_per_token_group_cast_ue8m0_scales():
    from oracle import quant
    # amax/448 already a power of two stays; anything above it goes to the next power
    t = np.array([1.0, 0.75, 3.0, 2.0 ** -20, 1.5 * 2.0 ** 10, 0.0, np.nextafter(np.float32(4.0), np.float32(5.0))],
                 dtype=np.float32)
    want = np.array([1.0, 1.0, 4.0, 2.0 ** -20, 2.0 ** 11, 1.0, 8.0], dtype=np.float32)
    assert np.array_equal(quant.pow2_ceil(t), want)
    rng = np.random.default_rng(33)
    x = (rng.standard_normal((3, 384)) * np.exp(rng.uniform(-10, 10, (3, 1)))).astype(np.float32)
    q, s = quant.per_token_group_cast(x, ue8m0=True)
    q32, s32 = quant.per_token_group_cast(x)
    assert np.all(s >= s32) and np.all(s < 2 * s32)                       # the next power of two
    assert np.array_equal(codecs.ue8m0_decode(codecs.ue8m0_encode(s)), s.astype(np.float64))  # exact in UE8M0
    assert np.all(np.abs(codecs.e4m3_decode(q)) <= 448)


def test_k_grouped_brute_force_exact():
    """K-grouped oracle against exact rational arithmetic written from the definition: each
    group sums the scaled products of its own K range only, into its own output, on top of
    its own C (an empty group returns C)."""
    from fractions import Fraction
    rng = np.random.default_rng(71)
    M, N, ks = 2, 3, [128, 0, 256, 128]
    K = sum(ks)
    a = rng.integers(0, 256, (M, K), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x30          # no NaN codes
    b[(b & 0x7F) == 0x7F] = 0x30
    sa = np.exp2(rng.uniform(-6, 2, (M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.uniform(-6, 2, (N, K // 128))).astype(np.float32)
    c = rng.standard_normal((len(ks), M, N)).astype(np.float32)
    A, B = oracle.e4m3_decode(a), oracle.e4m3_decode(b)
    got = oracle.k_grouped(a, sa, b, sb, ks, c)
    k0 = 0
    for g, kg in enumerate(ks):
        for i in range(M):
            for j in range(N):
                exact = Fraction(float(c[g, i, j]))
                mag = abs(exact)
                for k in range(k0, k0 + kg):
                    t = Fraction(float(sa[i, k // 128])) * Fraction(float(sb[j, k // 128])) * \
                        Fraction(float(A[i, k])) * Fraction(float(B[j, k]))
                    exact += t
                    mag += abs(t)
                assert abs(Fraction(float(got[g, i, j])) - exact) <= Fraction(1, 10 ** 14) * mag, (g, i, j)
        k0 += kg
    assert np.array_equal(got[1], c[1].astype(np.float64))          # the empty group is C itself


def test_k_grouped_single_group_is_the_dense_product():
    """One group covering all of K is the dense NT product with per-row scales on both sides
    (a special case that reduces to the pinned dense reference), and permuting the groups
    permutes the outputs."""
    rng = np.random.default_rng(72)
    M, N, K = 5, 7, 512
    a = (rng.integers(0, 0x7E, (M, K)) | (rng.integers(0, 2, (M, K)) << 7)).astype(np.uint8)
    b = (rng.integers(0, 0x7E, (N, K)) | (rng.integers(0, 2, (N, K)) << 7)).astype(np.uint8)
    sa = rng.uniform(0.01, 1, (M, 4)).astype(np.float32)
    sb = rng.uniform(0.01, 1, (N, 4)).astype(np.float32)
    c = rng.standard_normal((1, M, N)).astype(np.float32)
    d = oracle.k_grouped(a, sa, b, sb, [K], c)
    assert np.array_equal(d[0], oracle.gemm_nt(a, sa, b, sb, 1, c=c[0]))
    # two groups [256, 256] vs the same groups swapped: outputs swap
    c2 = rng.standard_normal((2, M, N)).astype(np.float32)
    d2 = oracle.k_grouped(a, sa, b, sb, [256, 256], c2)
    sw = lambda x: np.concatenate([x[:, 256:], x[:, :256]], axis=1)
    sws = lambda s: np.concatenate([s[:, 2:], s[:, :2]], axis=1)
    d3 = oracle.k_grouped(sw(a), sws(sa), sw(b), sws(sb), [256, 256], c2[::-1])
    assert np.array_equal(d2, d3[::-1])
    # the two halves of K add up to the whole, up to the rounding of the sum
    z = np.zeros((2, M, N), dtype=np.float32)
    halves = oracle.k_grouped(a, sa, b, sb, [256, 256], z)
    whole = oracle.k_grouped(a, sa, b, sb, [K], z[:1])[0]
    assert np.allclose(halves[0] + halves[1], whole, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- FP8 activations x FP4 weights
def test_e2m1_hand_values():
    """The sixteen E2M1 (OCP MX FP4) values: 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    t = codecs.e2m1_decode_table()
    assert t.tolist() == want
    assert np.signbit(t[8]) and not np.signbit(t[0])
    # every E2M1 value is exactly an E4M3 value (so FP4 weights widen to FP8 losslessly)
    e4 = codecs.e4m3_decode_table()
    assert all(v in e4 for v in want)


def test_unpack_fp4_hand_example():
    # byte 0x21: element 0 = low nibble 1 (0.5), element 1 = high nibble 2 (1.0);
    # byte 0xF7: element 2 = 7 (6.0), element 3 = 15 (-6.0); an odd K drops the last nibble
    codes = codecs.unpack_fp4(np.array([[0x21, 0xF7]], np.uint8), 4)
    assert codes.tolist() == [[1, 2, 7, 15]]
    assert codecs.e2m1_decode(codes).tolist() == [[0.5, 1.0, 6.0, -6.0]]
    assert codecs.unpack_fp4(np.array([[0x21, 0xF7]], np.uint8), 3).tolist() == [[1, 2, 7]]


def test_fp4_generator_encoder_is_nearest_ties_to_even():
    """The test generator's E2M1 encoder (the upstream quantizer, not the oracle): nearest
    value, ties to the even code, on every midpoint and on random values."""
    pos = codecs.e2m1_decode_table()[:8]
    mids = (pos[1:] + pos[:-1]) / 2
    got = gen.e2m1_codes(mids)
    # at a midpoint the two neighbours are codes i and i+1: the even one wins
    assert got.tolist() == [i if i % 2 == 0 else i + 1 for i in range(7)]
    x = np.random.default_rng(0).uniform(-7, 7, 10000)
    c = gen.e2m1_codes(x)
    d = np.abs(codecs.e2m1_decode(c) - np.clip(x, -6, 6))
    best = np.min(np.abs(np.concatenate([pos, -pos])[None, :] - np.clip(x, -6, 6)[:, None]), axis=1)
    assert np.array_equal(d, best)


def _fp8_fp4_brute(a, sa, b_packed, sb, K):
    t8 = [Fraction(v) if np.isfinite(v) else None for v in codecs.e4m3_decode_table()]
    t4 = [Fraction(v) for v in codecs.e2m1_decode_table()]
    codes = codecs.unpack_fp4(b_packed, K)
    M, N = a.shape[0], codes.shape[0]
    out = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(sa[i, k // 128])) * Fraction(float(sb[j, k // 32])) * t8[a[i, k]] * t4[codes[j, k]]
            out[i, j] = float(acc)
    return out


@pytest.mark.parametrize("K", [128, 256])
def test_fp8_fp4_gemm_vs_brute_force(K):
    """Exact rationals on tiny inputs: every E4M3 code (subnormals, +-448 included), every
    E2M1 code, power-of-two and arbitrary FP32 scales."""
    rng = np.random.default_rng(K)
    M, N = 5, 6
    a = rng.choice(np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8), (M, K))
    a[0, :4] = [0x7E, 0xFE, 0x01, 0x81]
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    b = gen.pack_fp4(codes)
    sa = rng.uniform(0.01, 2.0, (M, K // 128)).astype(np.float32)
    sb = np.exp2(rng.integers(-6, 3, (N, K // 32))).astype(np.float32)
    sb[1] = rng.uniform(0.01, 2.0, K // 32).astype(np.float32)
    D = gemm.gemm_fp8_fp4_nt(a, sa, b, sb)
    want = _fp8_fp4_brute(a, sa, b, sb, K)
    assert np.allclose(D, want, rtol=2.0 ** -48, atol=0)


def test_fp8_fp4_reduces_to_the_fp8_gemm():
    """With the four 32-long weight scales of every 128-long block equal, the FP8 x FP4 GEMM is
    the FP8 GEMM of the same values (E2M1 values are E4M3 values) with per-row weight scales:
    bitwise equal with power-of-two scales, where every step is exact."""
    p = gen.fp8_fp4(40, 72, 512, seed=3)
    sb128 = p["sb"].reshape(72, 4, 4)[:, :, 0]                      # one scale per 128 block
    sb = np.repeat(sb128, 4, axis=1)
    D4 = gemm.gemm_fp8_fp4_nt(p["a"], p["sa"], p["b"], sb)
    vals = codecs.e2m1_decode(codecs.unpack_fp4(p["b"], 512))
    e4 = codecs.e4m3_decode_table()
    lut = {float(v): c for c, v in enumerate(e4) if not np.isnan(v) and (c != 0x80)}
    b8 = np.vectorize(lambda v: lut[float(v)])(vals).astype(np.uint8)
    D8 = gemm.gemm_nt(p["a"], p["sa"], b8, sb128, 1)
    assert np.array_equal(D4, D8)


def test_fp8_fp4_sub_block_scale_linearity():
    """Doubling the weight scale of one 32-long block of one row adds exactly that block's
    contribution to that output column, and changes nothing else."""
    p = gen.fp8_fp4(16, 24, 256, seed=5)
    D = gemm.gemm_fp8_fp4_nt(p["a"], p["sa"], p["b"], p["sb"])
    sb2 = p["sb"].copy()
    sb2[7, 5] *= 2
    D2 = gemm.gemm_fp8_fp4_nt(p["a"], p["sa"], p["b"], sb2)
    A = codecs.e4m3_decode(p["a"])
    B = codecs.e2m1_decode(codecs.unpack_fp4(p["b"], 256))
    contrib = p["sa"][:, 1].astype(np.float64) * float(p["sb"][7, 5]) * (A[:, 160:192] @ B[7, 160:192])
    assert np.array_equal(D2[:, 7] - D[:, 7], contrib)
    assert np.array_equal(np.delete(D2, 7, axis=1), np.delete(D, 7, axis=1))


def test_fp8_fp4_dequantize_then_matmul():
    """The dequantize-then-matmul formulation (page "LinearQaunt-分块量化矩阵乘法"), with the
    weight scale expanded per 32 along K: agrees to float64 rounding."""
    p = gen.fp8_fp4(33, 50, 384, seed=6, with_c=True)
    A = codecs.e4m3_decode(p["a"]) * np.repeat(p["sa"].astype(np.float64), 128, axis=1)
    B = codecs.e2m1_decode(codecs.unpack_fp4(p["b"], 384)) * np.repeat(p["sb"].astype(np.float64), 32, axis=1)
    D = gemm.gemm_fp8_fp4_nt(p["a"], p["sa"], p["b"], p["sb"], c=p["c"])
    assert np.allclose(D, p["c"] + A @ B.T, rtol=1e-13, atol=1e-13)


def test_fp8_fp4_points_and_grouped_forms():
    """The point evaluator equals the full product; the grouped forms equal per-group dense
    products on their rows."""
    p = gen.fp8_fp4(30, 40, 256, seed=7, with_c=True)
    D, T = gemm.gemm_fp8_fp4_nt(p["a"], p["sa"], p["b"], p["sb"], c=p["c"], want_abs=True)
    ii, jj = np.array([0, 29, 5, 17]), np.array([0, 39, 22, 3])
    Dp, Tp = gemm.gemm_fp8_fp4_nt_points(p["a"], p["sa"], p["b"], p["sb"], ii, jj, c=p["c"])
    assert np.allclose(Dp, D[ii, jj], rtol=1e-14) and np.allclose(Tp, T[ii, jj], rtol=1e-14)
    q = gen.fp8_fp4_grouped_contiguous(3, 20, 256, seed=8, m_units=(1, 1), unit=8)
    lay = q["layout"].copy()
    lay[3] = -1
    Dc = gemm.grouped_contiguous_fp8_fp4(q["a"], q["sa"], q["b"], q["sb"], lay)
    assert np.isnan(Dc[3]).all()
    for g in range(3):
        rows = np.nonzero(lay == g)[0]
        assert np.array_equal(Dc[rows], gemm.gemm_fp8_fp4_nt(q["a"][rows], q["sa"][rows], q["b"][g], q["sb"][g]))
    r = gen.fp8_fp4_grouped_masked(3, 10, 20, 256, seed=9)
    mm = np.array([0, 10, 4], np.int32)
    Dm = gemm.grouped_masked_fp8_fp4(r["a"], r["sa"], r["b"], r["sb"], mm)
    assert np.isnan(Dm[0]).all() and np.isnan(Dm[2, 4:]).all()
    assert np.array_equal(Dm[2, :4], gemm.gemm_fp8_fp4_nt(r["a"][2, :4], r["sa"][2, :4], r["b"][2], r["sb"][2]))


# ---------------------------------------------------------------- operand layouts
def _brute_layout(layout, a_st, sa, b_st, sb, gran_n, c):
    """Exact value of D = C + op(A) @ op(B) written with the stored index of every operand
    element: A[i, k] is a_st[i, k] for an "n" A and a_st[k, i] for a "t" A; B's element of
    output column j at depth k is b_st[j, k] for a "t" B and b_st[k, j] for an "n" B."""
    t = codecs.e4m3_decode_table()
    M = a_st.shape[0] if layout[0] == "n" else a_st.shape[1]
    K = a_st.shape[1] if layout[0] == "n" else a_st.shape[0]
    N = b_st.shape[0] if layout[1] == "t" else b_st.shape[1]
    D = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            acc = Fraction(float(c[i, j]))
            for k in range(K):
                av = a_st[i, k] if layout[0] == "n" else a_st[k, i]
                bv = b_st[j, k] if layout[1] == "t" else b_st[k, j]
                acc += (Fraction(float(sa[i, k // 128])) * Fraction(float(sb[j // gran_n, k // 128])) *
                        Fraction(float(t[av])) * Fraction(float(t[bv])))
            D[i, j] = float(acc)
    return D


@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
@pytest.mark.parametrize("gran_n", [128, 1])
def test_gemm_layouts_vs_brute_force(layout, gran_n):
    """Every layout against exact arithmetic on the stored operands; M, N and K all differ, so
    reading an operand through the wrong storage changes the shape or the values."""
    rng = np.random.default_rng(100 + 7 * len(layout) + gran_n + ord(layout[0]) + 3 * ord(layout[1]))
    M, N, K = 3, 5, 256
    a, sa, b, sb = _random_tiny(rng, M, N, K, gran_n)
    a_st = a if layout[0] == "n" else np.ascontiguousarray(a.T)
    b_st = b if layout[1] == "t" else np.ascontiguousarray(b.T)
    c = rng.standard_normal((M, N)).astype(np.float32)
    D, T = oracle.gemm_layout(layout, a_st, sa, b_st, sb, gran_n, c=c, want_abs=True)
    assert D.shape == (M, N)
    Dx = _brute_layout(layout, a_st, sa, b_st, sb, gran_n, c)
    assert np.all(np.abs(D - Dx) <= 2.0 ** -48 * (T + np.abs(c)))
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Dp, _ = oracle.gemm_layout_points(layout, a_st, sa, b_st, sb, ii.ravel(), jj.ravel(), gran_n, c=c)
    assert np.all(np.abs(Dp - Dx.ravel()) <= 2.0 ** -48 * (T.ravel() + np.abs(c).ravel()))


def test_gemm_layout_transpose_is_not_the_identity():
    """A square stored A (M = K = 128) that is not symmetric: reading it under "tt" differs
    from reading it under "nt", and "tt" on its transpose is "nt" on it."""
    rng = np.random.default_rng(5)
    a, sa, b, sb = _random_tiny(rng, 128, 4, 128, 1)
    d_nt = oracle.gemm_layout("nt", a, sa, b, sb, 1)
    d_tt = oracle.gemm_layout("tt", a, sa, b, sb, 1)
    assert not np.allclose(d_nt, d_tt)
    assert np.array_equal(d_nt, oracle.gemm_layout("tt", np.ascontiguousarray(a.T), sa, b, sb, 1))


def test_grouped_contiguous_nn_vs_brute_force():
    rng = np.random.default_rng(19)
    G, N, K = 2, 5, 256
    rows = np.array([1, 1, -1, 0, 0, 0], dtype=np.int32)
    a, sa, _, _ = _random_tiny(rng, len(rows), 1, K, 128)
    b = np.stack([np.ascontiguousarray(_random_tiny(rng, 1, N, K, 128)[2].T) for _ in range(G)])  # [G, K, N]
    sb = np.stack([_random_tiny(rng, 1, N, K, 128)[3] for _ in range(G)])
    D = oracle.grouped_contiguous_nn(a, sa, b, sb, rows)
    for i, g in enumerate(rows):
        if g < 0:
            assert np.isnan(D[i]).all()
            continue
        Dx = _brute_layout("nn", a[i:i + 1], sa[i:i + 1], b[g], sb[g], 128, np.zeros((1, N)))
        assert np.allclose(D[i], Dx[0], rtol=1e-13, atol=0)


def test_k_grouped_tn_vs_brute_force():
    """K-grouped with token-major operands (A [sum K, M], B [sum K, N]): each group sums its own
    K range of the stored rows into its own output on top of its C."""
    rng = np.random.default_rng(23)
    M, N, ks = 3, 2, [128, 256, 0]
    K = sum(ks)
    a_st = rng.integers(0, 256, (K, M), dtype=np.uint8)
    b_st = rng.integers(0, 256, (K, N), dtype=np.uint8)
    a_st[(a_st & 0x7F) == 0x7F] = 0x31
    b_st[(b_st & 0x7F) == 0x7F] = 0x31
    sa = np.exp2(rng.uniform(-4, 2, (M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.uniform(-4, 2, (N, K // 128))).astype(np.float32)
    c = rng.standard_normal((len(ks), M, N)).astype(np.float32)
    got = oracle.k_grouped_tn(a_st, sa, b_st, sb, ks, c)
    t = codecs.e4m3_decode_table()
    k0 = 0
    for g, kg in enumerate(ks):
        for i in range(M):
            for j in range(N):
                exact, mag = Fraction(float(c[g, i, j])), abs(Fraction(float(c[g, i, j])))
                for k in range(k0, k0 + kg):
                    p = (Fraction(float(sa[i, k // 128])) * Fraction(float(sb[j, k // 128])) *
                         Fraction(float(t[a_st[k, i]])) * Fraction(float(t[b_st[k, j]])))
                    exact += p
                    mag += abs(p)
                assert abs(Fraction(float(got[g, i, j])) - exact) <= Fraction(1, 10 ** 14) * mag
        k0 += kg


def test_fp8_fp4_tt_vs_brute_force():
    """FP8 x FP4 with A stored [K, M]: exact sum over the stored activations and the packed
    weight nibbles (low nibble = even K), each 32-long group with its own weight scale."""
    rng = np.random.default_rng(29)
    M, N, K = 3, 4, 256
    a_st = rng.integers(0, 256, (K, M), dtype=np.uint8)
    a_st[(a_st & 0x7F) == 0x7F] = 0x2A
    b = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = np.exp2(rng.integers(-3, 3, (M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-3, 3, (N, K // 32))).astype(np.float32)
    got = oracle.gemm_fp8_fp4_tt(a_st, sa, b, sb)
    t8, t4 = codecs.e4m3_decode_table(), codecs.e2m1_decode_table()
    for i in range(M):
        for j in range(N):
            exact = Fraction(0)
            for k in range(K):
                nib = (b[j, k // 2] >> (4 * (k % 2))) & 0xF
                exact += (Fraction(float(sa[i, k // 128])) * Fraction(float(sb[j, k // 32])) *
                          Fraction(float(t8[a_st[k, i]])) * Fraction(float(t4[nib])))
            assert Fraction(float(got[i, j])) == exact        # every partial and sum is exact here
