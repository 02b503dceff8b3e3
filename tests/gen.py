"""Seeded synthetic inputs for block-scaled FP8 GEMM (shared by the oracle side
and the HIP side of every test and by bench.py).

This module holds none of the GEMM's arithmetic: it only draws random numbers
and quantizes them the way an upstream cast kernel would (the library itself
never quantizes; page "02 · DeepGEMM 技术解析" §1.1 says the FP8 cast is the
caller's job).  Quantization recipe (page "02 · DeepGEMM 技术解析" §1.1):
one FP32 scale per 1x128 K group of activations and per 128x128 block of
weights, scale = amax / 448 (1 when the group is all zero), codes =
round-to-nearest-even E4M3 of x / scale clamped to +-448, using torch's
``float8_e4m3fn`` cast (a library routine; the clamp is needed because that
cast turns values of 464 and above into NaN instead of saturating).

Every generator takes a seed and draws, in this order, from one numpy PCG64
stream: A, A outliers, B, C, group sizes, scales.  Arrays are numpy:
E4M3 codes as uint8, scales as float32 in their plain (K-major) layout:
``sa[M, sf_k]``, ``sb[ceil(N/128), sf_k]``.
"""
import numpy as np
import torch

BLOCK = 128
E4M3_MAX = 448.0


def _cdiv(a, b):
    return (a + b - 1) // b


def e4m3_codes(x):
    """float32 array -> E4M3 codes (uint8) by torch's RNE cast after clamping to +-448."""
    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def quantize_act(x):
    """Activations [M, K] -> (codes [M, K] uint8, scales [M, ceil(K/128)] float32), 1x128 groups."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    sf_k = _cdiv(K, BLOCK)
    xp = np.zeros((M, sf_k * BLOCK), dtype=np.float32)
    xp[:, :K] = x
    amax = np.abs(xp.reshape(M, sf_k, BLOCK)).max(axis=2)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s[amax == 0] = 1.0
    q = xp.reshape(M, sf_k, BLOCK) / s[:, :, None]
    return e4m3_codes(q.reshape(M, -1)[:, :K]), s


def quantize_weight(x):
    """Weights [N, K] -> (codes [N, K] uint8, scales [ceil(N/128), ceil(K/128)] float32), 128x128 blocks."""
    x = np.asarray(x, dtype=np.float32)
    N, K = x.shape
    nb, sf_k = _cdiv(N, BLOCK), _cdiv(K, BLOCK)
    xp = np.zeros((nb * BLOCK, sf_k * BLOCK), dtype=np.float32)
    xp[:N, :K] = x
    blk = xp.reshape(nb, BLOCK, sf_k, BLOCK)
    amax = np.abs(blk).max(axis=(1, 3))
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s[amax == 0] = 1.0
    q = (blk / s[:, None, :, None]).reshape(nb * BLOCK, sf_k * BLOCK)
    return e4m3_codes(q[:N, :K]), s


def _act_values(rng, M, K, outliers=True):
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers and M * K > 0:
        n = int(round(0.001 * M * K))
        pos = rng.choice(M * K, size=n, replace=False)
        x.reshape(-1)[pos] *= np.float32(50.0)
    return x


def dense(M, N, K, seed=0, a_std=1.0, b_std=0.02, outliers=True, with_c=False):
    """Dense NT problem with V3-style data: A ~ N(0, a_std) with 0.1% outliers x50,
    B ~ N(0, b_std); optional C ~ N(0, 1) float32 [M, N]."""
    rng = np.random.default_rng(seed)
    xa = _act_values(rng, M, K, outliers) * np.float32(a_std)
    xb = rng.standard_normal((N, K), dtype=np.float32) * np.float32(b_std)
    c = rng.standard_normal((M, N), dtype=np.float32) if with_c else None
    a, sa = quantize_act(xa)
    b, sb = quantize_weight(xb)
    return dict(a=a, sa=sa, b=b, sb=sb, c=c, M=M, N=N, K=K)


def tiny_dense(seed=0):
    """M=128, N=256, K=512; A, B ~ N(0, 1); amax/448 scales; no C."""
    return dense(128, 256, 512, seed=seed, a_std=1.0, b_std=1.0, outliers=False)


def pow2_exact(M, N, K, seed=0, with_c=False):
    """Inputs whose every FP32 partial sum is exact: payloads are integers in
    [-8, 8] (exact E4M3 codes) and scales are 2^e with e in [-3, 0]."""
    rng = np.random.default_rng(seed)
    xa = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    xb = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    c = None
    if with_c:
        c = (rng.integers(-64, 65, size=(M, N)).astype(np.float32) / np.float32(64.0))
    sa = np.exp2(rng.integers(-3, 1, size=(M, _cdiv(K, BLOCK)))).astype(np.float32)
    sb = np.exp2(rng.integers(-3, 1, size=(_cdiv(N, BLOCK), _cdiv(K, BLOCK)))).astype(np.float32)
    return dict(a=e4m3_codes(xa), sa=sa, b=e4m3_codes(xb), sb=sb, c=c, M=M, N=N, K=K)


def grouped_contiguous(G, N, K, seed=0, m_units=(1, 8), unit=BLOCK, b_std=0.02):
    """M-grouped contiguous MoE problem: group sizes M_g = unit * U{m_units},
    rows concatenated by group, B [G, N, K] with 128x128 scales, and the int32
    row -> group vector."""
    rng = np.random.default_rng(seed)
    # group sizes are drawn first so that A's shape is known; order documented above
    sizes = rng.integers(m_units[0], m_units[1] + 1, size=G) * unit
    Mt = int(sizes.sum())
    xa = _act_values(rng, Mt, K, True)
    a, sa = quantize_act(xa)
    del xa
    b = np.empty((G, N, K), dtype=np.uint8)
    sb = np.empty((G, _cdiv(N, BLOCK), _cdiv(K, BLOCK)), dtype=np.float32)
    for g in range(G):
        xb = rng.standard_normal((N, K), dtype=np.float32) * np.float32(b_std)
        b[g], sb[g] = quantize_weight(xb)
    layout = np.repeat(np.arange(G, dtype=np.int32), sizes)
    return dict(a=a, sa=sa, b=b, sb=sb, layout=layout, sizes=sizes, G=G, N=N, K=K, M=Mt)


def grouped_masked(G, M_max, N, K, seed=0, pow2_scales=True):
    """M-grouped masked decode problem: A [G, M_max, K], B [G, N, K], valid rows
    per group m_g ~ U{0..M_max}.  Payloads are E4M3_RNE(N(0, 1)); with
    ``pow2_scales`` every scale is 2^e, e ~ U{-8..0}, drawn per A 1x128 group and
    per B 128x128 block (otherwise amax/448 scales)."""
    rng = np.random.default_rng(seed)
    sf_k, nb = _cdiv(K, BLOCK), _cdiv(N, BLOCK)
    xa = rng.standard_normal((G, M_max, K), dtype=np.float32)
    b = np.empty((G, N, K), dtype=np.uint8)
    sb = np.empty((G, nb, sf_k), dtype=np.float32)
    xbs = []
    for g in range(G):
        xbs.append(rng.standard_normal((N, K), dtype=np.float32))
    masked_m = rng.integers(0, M_max + 1, size=G).astype(np.int32)
    if pow2_scales:
        a = e4m3_codes(xa.reshape(G * M_max, K)).reshape(G, M_max, K)
        sa = np.exp2(rng.integers(-8, 1, size=(G, M_max, sf_k))).astype(np.float32)
        for g in range(G):
            b[g] = e4m3_codes(xbs[g])
        sb[:] = np.exp2(rng.integers(-8, 1, size=(G, nb, sf_k))).astype(np.float32)
    else:
        a, sa = quantize_act(xa.reshape(G * M_max, K))
        a = a.reshape(G, M_max, K)
        sa = sa.reshape(G, M_max, sf_k)
        for g in range(G):
            b[g], sb[g] = quantize_weight(xbs[g])
    return dict(a=a, sa=sa, b=b, sb=sb, masked_m=masked_m, G=G, M_max=M_max, N=N, K=K)


# The five workloads (sizes as stated for the V3-shaped benchmark set).
def config1(seed=0):
    return tiny_dense(seed)


def config2(seed=0, M=4096):
    return dense(M, 7168, 2048, seed=seed)


def config3(seed=0):
    return dense(4096, 1536, 7168, seed=seed, with_c=True)


def config4(seed=0):
    return grouped_contiguous(32, 4096, 7168, seed=seed)


def config5(seed=0):
    return grouped_masked(32, 256, 7168, 2048, seed=seed, pow2_scales=True)


def k_grouped(m, n, ks, seed=0):
    """K-grouped weight-gradient problem: both operands are activation-like ([m, sum ks] and
    [n, sum ks], N(0, 1) with x50 outliers quantized in 1x128 groups along K, so both carry
    one scale per row and K block), and a C term [G, m, n] of N(0, 1)."""
    rng = np.random.default_rng(seed)
    K = int(sum(ks))
    xa = rng.standard_normal((m, K), dtype=np.float32)
    xb = rng.standard_normal((n, K), dtype=np.float32)
    for x in (xa, xb):
        if x.size:
            idx = rng.choice(x.size, size=max(1, x.size // 1000), replace=False)
            x.reshape(-1)[idx] *= np.float32(50.0)
    a, sa = quantize_act(xa) if K else (np.zeros((m, 0), np.uint8), np.zeros((m, 0), np.float32))
    b, sb = quantize_act(xb) if K else (np.zeros((n, 0), np.uint8), np.zeros((n, 0), np.float32))
    c = rng.standard_normal((len(ks), m, n), dtype=np.float32)
    return dict(a=a, sa=sa, b=b, sb=sb, c=c, ks=list(ks), m=m, n=n)


# ---------------------------------------------------------------- FP8 activations x FP4 weights
E2M1_MAX = 6.0
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_codes(x):
    """float array -> E2M1 codes (uint8, 0..15): nearest of the eight magnitudes (ties to the
    even code, i.e. the even mantissa), clamped to +-6, sign in bit 3 (zero is +0)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), E2M1_MAX)
    hi = np.clip(np.searchsorted(_E2M1_POS, ax), 1, 7)
    lo = hi - 1
    dlo, dhi = ax - _E2M1_POS[lo], _E2M1_POS[hi] - ax
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    sign = ((x < 0) & (pick > 0)).astype(np.uint8) << np.uint8(3)
    return (pick.astype(np.uint8) | sign)


def pack_fp4(codes):
    """codes [..., K] (K even) -> bytes [..., K/2], element 2t in the low nibble of byte t."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)


def pow2_ceil_scale(amax, qmax):
    """Power-of-two scale for a group: the FP32 amax / qmax raised to the next power of two
    (1 for an all-zero group), so every quotient stays within +-qmax (a UE8M0 scale)."""
    s = (np.asarray(amax, dtype=np.float32) / np.float32(qmax)).astype(np.float32)
    m, e = np.frexp(s.astype(np.float64))
    p = np.where(m == 0.5, s, np.ldexp(1.0, e)).astype(np.float32)
    return np.where(s == 0, np.float32(1.0), p).astype(np.float32)


def quantize_act_pow2(x):
    """Activations [M, K] -> (E4M3 codes, power-of-two scales [M, K/128]), 1x128 groups."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    g = x.reshape(M, K // BLOCK, BLOCK)
    s = pow2_ceil_scale(np.abs(g).max(axis=2), E4M3_MAX)
    return e4m3_codes((g / s[:, :, None]).reshape(M, K)), s


def quantize_weight_fp4(x):
    """Weights [N, K] -> (packed E2M1 bytes [N, K/2], power-of-two scales [N, K/32]), one
    scale per row and 32-long K group (the V4 routed-expert weight recipe)."""
    x = np.asarray(x, dtype=np.float32)
    N, K = x.shape
    g = x.reshape(N, K // 32, 32)
    s = pow2_ceil_scale(np.abs(g).max(axis=2), E2M1_MAX)
    return pack_fp4(e2m1_codes((g / s[:, :, None]).reshape(N, K))), s


def fp8_fp4(M, N, K, seed=0, b_std=0.02, with_c=False):
    """Dense FP8 x FP4 problem: A ~ N(0,1) with 0.1% x50 outliers (E4M3, 1x128 power-of-two
    scales), B ~ N(0, b_std) (E2M1, 1x32 power-of-two scales), optional C ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    xa = _act_values(rng, M, K, True)
    xb = rng.standard_normal((N, K), dtype=np.float32) * np.float32(b_std)
    c = rng.standard_normal((M, N), dtype=np.float32) if with_c else None
    a, sa = quantize_act_pow2(xa)
    b, sb = quantize_weight_fp4(xb)
    return dict(a=a, sa=sa, b=b, sb=sb, c=c, M=M, N=N, K=K)


def fp8_fp4_grouped_contiguous(G, N, K, seed=0, m_units=(1, 8), unit=BLOCK):
    rng = np.random.default_rng(seed)
    sizes = rng.integers(m_units[0], m_units[1] + 1, size=G) * unit
    Mt = int(sizes.sum())
    a, sa = quantize_act_pow2(_act_values(rng, Mt, K, True))
    b = np.empty((G, N, K // 2), dtype=np.uint8)
    sb = np.empty((G, N, K // 32), dtype=np.float32)
    for g in range(G):
        b[g], sb[g] = quantize_weight_fp4(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    layout = np.repeat(np.arange(G, dtype=np.int32), sizes)
    return dict(a=a, sa=sa, b=b, sb=sb, layout=layout, sizes=sizes, G=G, N=N, K=K, M=Mt)


def fp8_fp4_grouped_masked(G, M_max, N, K, seed=0):
    rng = np.random.default_rng(seed)
    a, sa = quantize_act_pow2(_act_values(rng, G * M_max, K, True))
    b = np.empty((G, N, K // 2), dtype=np.uint8)
    sb = np.empty((G, N, K // 32), dtype=np.float32)
    for g in range(G):
        b[g], sb[g] = quantize_weight_fp4(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    masked_m = rng.integers(0, M_max + 1, size=G).astype(np.int32)
    return dict(a=a.reshape(G, M_max, K), sa=sa.reshape(G, M_max, K // BLOCK), b=b, sb=sb, masked_m=masked_m,
                G=G, M_max=M_max, N=N, K=K)
