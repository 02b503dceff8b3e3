"""Float64 references for block-scaled FP8 GEMM, D = C + A @ B^T.  Test infrastructure only.

Follows the plain definition on the pages:
  * page "02 · DeepGEMM 技术解析" §2.2: per 128-long K block the low-precision
    partial is multiplied by scale_a * scale_b and added into an FP32 final
    accumulator that starts at 0; §1.1: activations carry one FP32 scale per
    1x128 K group, weights one per 128x128 block.
  * page "第13章 DeepGEMM" §13.3: ``fp8_gemm_nt`` computes D = C + A @ B.T with A
    row-major [M, K] and B stored [N, K]; the algorithm box accumulates
    ``scale_x * scale_w * (x_block @ w_block.T)`` per K tile.
  * page "第13章 DeepGEMM" §13.6: M-grouped GEMM is the per-expert loop
    ``y[idx] += expert(x[idx])`` with only M grouped (N and K fixed).
  * page "02 · DeepGEMM 技术解析" §5.2: the masked layout computes only the
    valid rows of each group.

Each block partial ``P_b = dec(A_b) @ dec(B_b)^T`` is exact in float64 whatever
order the library matmul sums it in: every product of two E4M3 values is a
multiple of 2^-18 below 2^18, so any partial sum of up to 2^13 of them is an
integer number of 2^-18 units below 2^53.  The FP32 scale product is exact in
float64 (24 + 24 significand bits); ``(sa * sb) * P_b`` and the sum over
blocks round once each.

The scale arguments are the plain logical layouts (not the MN-major device
layout): ``sa[i, b]`` per row and K block, ``sb[jb, b]`` per weight block
(``jb = j // gran_n``; ``gran_n`` is 128 for 128x128 weight blocks and 1 for
per-row weight scales).  K need not be a multiple of 128: the last block is
then shorter.
"""
import numpy as np

from .codecs import e4m3_decode, e2m1_decode, unpack_fp4

BLOCK_K = 128


def _sf_k(K):
    return (K + BLOCK_K - 1) // BLOCK_K


def expand_scales_b(sb, N, gran_n):
    """Weight scales [ceil(N / gran_n), sf_k] -> one row per output column [N, sf_k]."""
    sb = np.asarray(sb, dtype=np.float64)
    return sb[np.arange(N) // gran_n]


def gemm_nt(a_codes, sa, b_codes, sb, gran_n=128, c=None, want_abs=False):
    """Dense NT reference.

    a_codes: uint8 [M, K] E4M3 codes; sa: [M, sf_k] scales (any float dtype).
    b_codes: uint8 [N, K]; sb: [ceil(N / gran_n), sf_k].
    c: None or [M, N].
    Returns D float64 [M, N]; with ``want_abs`` also T[i, j] = sum_k |A'_ik * B'_jk|
    (A', B' the dequantized values), which the tolerances are stated against.
    """
    A = e4m3_decode(a_codes)
    B = e4m3_decode(b_codes)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    sf_k = _sf_k(K)
    sa = np.asarray(sa, dtype=np.float64)
    assert sa.shape == (M, sf_k)
    sbe = expand_scales_b(sb, N, gran_n)
    assert sbe.shape == (N, sf_k)
    D = np.zeros((M, N), dtype=np.float64)
    T = np.zeros((M, N), dtype=np.float64) if want_abs else None
    for b in range(sf_k):
        ks = slice(b * BLOCK_K, min((b + 1) * BLOCK_K, K))
        P = A[:, ks] @ B[:, ks].T                      # exact block partial
        S = sa[:, b][:, None] * sbe[:, b][None, :]     # exact scale product
        D += S * P
        if want_abs:
            T += np.abs(S) * (np.abs(A[:, ks]) @ np.abs(B[:, ks]).T)
    if c is not None:
        D = np.asarray(c, dtype=np.float64) + D
    return (D, T) if want_abs else D


def gemm_nt_points(a_codes, sa, b_codes, sb, ii, jj, gran_n=128, c=None, chunk=4096):
    """The same definition evaluated only at output positions (ii[p], jj[p]).

    Returns (D, T) as float64 vectors.  Used for sampled checks at sizes where
    the full product would take too long.
    """
    ii = np.asarray(ii, dtype=np.int64)
    jj = np.asarray(jj, dtype=np.int64)
    K = a_codes.shape[1]
    sf_k = _sf_k(K)
    sa = np.asarray(sa, dtype=np.float64)
    sb = np.asarray(sb, dtype=np.float64)
    Kp = sf_k * BLOCK_K
    D = np.empty(len(ii), dtype=np.float64)
    T = np.empty(len(ii), dtype=np.float64)
    for s in range(0, len(ii), chunk):
        i = ii[s:s + chunk]
        j = jj[s:s + chunk]
        prod = np.zeros((len(i), Kp), dtype=np.float64)
        prod[:, :K] = e4m3_decode(a_codes[i]) * e4m3_decode(b_codes[j])
        blk = prod.reshape(len(i), sf_k, BLOCK_K)
        P = blk.sum(axis=2)                             # exact block partials
        Pabs = np.abs(blk).sum(axis=2)
        S = sa[i] * sb[j // gran_n]                     # [n, sf_k], exact
        D[s:s + chunk] = (S * P).sum(axis=1)
        T[s:s + chunk] = (np.abs(S) * Pabs).sum(axis=1)
    if c is not None:
        D = np.asarray(c, dtype=np.float64)[ii, jj] + D
    return D, T


def grouped_contiguous(a_codes, sa, b_codes, sb, grouped_layout, gran_n=128, want_abs=False):
    """M-grouped contiguous reference: rows of A concatenated by group.

    a_codes [sumM, K], sa [sumM, sf_k]; b_codes [G, N, K], sb [G, nb, sf_k];
    grouped_layout [sumM] int: the group of each row, negative = no output.
    Returns D [sumM, N] float64 with NaN in rows that produce no output.
    """
    gl = np.asarray(grouped_layout)
    G, N, _ = b_codes.shape
    M = a_codes.shape[0]
    D = np.full((M, N), np.nan)
    T = np.full((M, N), np.nan) if want_abs else None
    for g in range(G):                      # the per-expert loop
        idx = np.nonzero(gl == g)[0]
        if len(idx) == 0:
            continue
        r = gemm_nt(a_codes[idx], np.asarray(sa)[idx], b_codes[g], sb[g], gran_n,
                    want_abs=want_abs)
        if want_abs:
            D[idx], T[idx] = r
        else:
            D[idx] = r
    return (D, T) if want_abs else D


def grouped_masked(a_codes, sa, b_codes, sb, masked_m, gran_n=128, want_abs=False):
    """M-grouped masked reference: A [G, M_max, K]; only rows i < masked_m[g] are valid.

    sa [G, M_max, sf_k]; b_codes [G, N, K]; sb [G, nb, sf_k].
    masked_m[g] is clamped to [0, M_max].  Returns D [G, M_max, N] with NaN
    in rows that produce no output.
    """
    G, Mmax, _ = a_codes.shape
    N = b_codes.shape[1]
    D = np.full((G, Mmax, N), np.nan)
    T = np.full((G, Mmax, N), np.nan) if want_abs else None
    for g in range(G):
        m = int(min(max(int(masked_m[g]), 0), Mmax))
        if m == 0:
            continue
        r = gemm_nt(a_codes[g, :m], np.asarray(sa)[g, :m], b_codes[g], sb[g], gran_n,
                    want_abs=want_abs)
        if want_abs:
            D[g, :m], T[g, :m] = r
        else:
            D[g, :m] = r
    return (D, T) if want_abs else D


def k_grouped(a_codes, sa, b_codes, sb, ks, c, want_abs=False):
    """K-grouped contiguous reference (the MoE weight-gradient form: page "02 · DeepGEMM
    技术解析" §3.3 and page "第13章 DeepGEMM" §13.6 and §13.13): M and N are fixed, the
    groups are concatenated along K, and group g accumulates its own K range into its
    own output, starting from the required C term:

        D[g] = C[g] + sum_{b in group g's K blocks} sa[:, b] * sb[:, b] * P_b

    a_codes [M, sum K], b_codes [N, sum K]; sa [M, sum sf_k], sb [N, sum sf_k] (one scale
    per row and 128-long K block on both sides, logical layout); ks: the K of each group,
    each a multiple of 128 (0 allowed: then D[g] = C[g]); c [G, M, N].  Returns D [G, M, N].
    """
    ks = [int(k) for k in ks]
    assert all(k >= 0 and k % BLOCK_K == 0 for k in ks)
    c = np.asarray(c, dtype=np.float64)
    G, M, N = c.shape
    assert len(ks) == G and a_codes.shape == (M, sum(ks)) and b_codes.shape == (N, sum(ks))
    D = c.copy()
    T = np.zeros((G, M, N)) if want_abs else None
    k0 = 0
    for g, k in enumerate(ks):              # one dense NT product per group
        if k:
            kr, br = slice(k0, k0 + k), slice(k0 // BLOCK_K, (k0 + k) // BLOCK_K)
            r = gemm_nt(a_codes[:, kr], np.asarray(sa)[:, br], b_codes[:, kr], np.asarray(sb)[:, br], 1,
                        c=c[g], want_abs=want_abs)
            if want_abs:
                D[g], T[g] = r
            else:
                D[g] = r
        k0 += k
    return (D, T) if want_abs else D


BLOCK_K_FP4 = 32


def gemm_fp8_fp4_nt(a_codes, sa, b_packed, sb, c=None, want_abs=False):
    """FP8 activations x FP4 weights, D = C + A @ B^T (page "第13章 DeepGEMM" §13.1: the V4
    routed-expert recipe, FP8 activations and FP4 weights with one weight scale per 32 K
    elements; §13.5: FP4 weights fed to the matrix unit together with FP8 activations, the
    scales applied inside the MMA; page "02 · DeepGEMM 技术解析" §3.1: the scales are UE8M0
    powers of two).

    a_codes: uint8 [M, K] E4M3 codes; sa: [M, ceil(K/128)] activation scales (one per row
    and 128-long K block).  b_packed: uint8 [N, ceil(K/2)] E2M1 codes, two per byte (low
    nibble first); sb: [N, ceil(K/32)] weight scales (one per row and 32-long K block).

        D[i, j] = C[i, j] + sum_b sa[i, b] * sum_{s in block b} sb[j, s] * P[i, j, s]
        P[i, j, s] = sum_{k in 32-block s} dec(A[i, k]) * dec(B[j, k])

    Every E4M3 x E2M1 product is a multiple of 2^-10 below 2^12 in magnitude, so each
    32-long partial P is exact in float64 in any order.  Returns D float64 [M, N] (and T,
    the sum of |A'_ik B'_jk| over the dequantized values, with ``want_abs``).
    """
    A = e4m3_decode(a_codes)
    M, K = A.shape
    B = e2m1_decode(unpack_fp4(b_packed, K))
    N = B.shape[0]
    sa = np.asarray(sa, dtype=np.float64)
    sb = np.asarray(sb, dtype=np.float64)
    assert sa.shape == (M, _sf_k(K))
    n_sub = (K + BLOCK_K_FP4 - 1) // BLOCK_K_FP4
    assert sb.shape == (N, n_sub)
    D = np.zeros((M, N), dtype=np.float64)
    T = np.zeros((M, N), dtype=np.float64) if want_abs else None
    for s in range(n_sub):
        ks = slice(s * BLOCK_K_FP4, min((s + 1) * BLOCK_K_FP4, K))
        b = (s * BLOCK_K_FP4) // BLOCK_K
        P = A[:, ks] @ B[:, ks].T                       # exact 32-long partial
        S = sa[:, b][:, None] * sb[:, s][None, :]       # exact scale product
        D += S * P
        if want_abs:
            T += np.abs(S) * (np.abs(A[:, ks]) @ np.abs(B[:, ks]).T)
    if c is not None:
        D = np.asarray(c, dtype=np.float64) + D
    return (D, T) if want_abs else D


def gemm_fp8_fp4_nt_points(a_codes, sa, b_packed, sb, ii, jj, c=None):
    """gemm_fp8_fp4_nt evaluated only at output positions (ii[p], jj[p]); returns (D, T)."""
    ii = np.asarray(ii, dtype=np.int64)
    jj = np.asarray(jj, dtype=np.int64)
    K = a_codes.shape[1]
    n_sub = (K + BLOCK_K_FP4 - 1) // BLOCK_K_FP4
    Kp = n_sub * BLOCK_K_FP4
    prod = np.zeros((len(ii), Kp), dtype=np.float64)
    prod[:, :K] = e4m3_decode(a_codes[ii]) * e2m1_decode(unpack_fp4(b_packed[jj], K))
    blk = prod.reshape(len(ii), n_sub, BLOCK_K_FP4)
    P, Pabs = blk.sum(axis=2), np.abs(blk).sum(axis=2)
    sa = np.asarray(sa, dtype=np.float64)[ii]
    S = sa[:, np.arange(n_sub) * BLOCK_K_FP4 // BLOCK_K] * np.asarray(sb, dtype=np.float64)[jj]
    D = (S * P).sum(axis=1)
    T = (np.abs(S) * Pabs).sum(axis=1)
    if c is not None:
        D = np.asarray(c, dtype=np.float64)[ii, jj] + D
    return D, T


def grouped_contiguous_fp8_fp4(a_codes, sa, b_packed, sb, grouped_layout, want_abs=False):
    """M-grouped contiguous FP8 x FP4 (page "第13章 DeepGEMM" §13.6: only M is grouped):
    row i uses group g = grouped_layout[i] >= 0, i.e. B[g] and sb[g]; negative rows produce no
    output (NaN).  b_packed [G, N, ceil(K/2)], sb [G, N, ceil(K/32)]."""
    gl = np.asarray(grouped_layout)
    G, N, _ = b_packed.shape
    D = np.full((a_codes.shape[0], N), np.nan)
    T = np.full_like(D, np.nan) if want_abs else None
    for g in range(G):                      # the per-expert loop
        idx = np.nonzero(gl == g)[0]
        if len(idx) == 0:
            continue
        r = gemm_fp8_fp4_nt(a_codes[idx], np.asarray(sa)[idx], b_packed[g], sb[g], want_abs=want_abs)
        if want_abs:
            D[idx], T[idx] = r
        else:
            D[idx] = r
    return (D, T) if want_abs else D


def grouped_masked_fp8_fp4(a_codes, sa, b_packed, sb, masked_m, want_abs=False):
    """M-grouped masked FP8 x FP4 (page "02 · DeepGEMM 技术解析" §5.2): A [G, M_max, K];
    rows i < clamp(masked_m[g], 0, M_max) of each group are computed, the others are NaN."""
    G, Mmax, _ = a_codes.shape
    N = b_packed.shape[1]
    D = np.full((G, Mmax, N), np.nan)
    T = np.full_like(D, np.nan) if want_abs else None
    for g in range(G):
        m = int(min(max(int(masked_m[g]), 0), Mmax))
        if m == 0:
            continue
        r = gemm_fp8_fp4_nt(a_codes[g, :m], np.asarray(sa)[g, :m], b_packed[g], sb[g], want_abs=want_abs)
        if want_abs:
            D[g, :m], T[g, :m] = r
        else:
            D[g, :m] = r
    return (D, T) if want_abs else D


# ---- operand layouts ---------------------------------------------------------------------
# Page "第13章 DeepGEMM" §13.3: the two suffix letters give the transposition state of A and
# B in D = C + A @ B, so fp8_gemm_nt is D = C + A @ B.T, and the family also has nn, tn and tt
# (the K-grouped weight-gradient form is named tn, §13.13; page "02 · DeepGEMM 技术解析" §5.1
# names an nn form of the M-grouped contiguous GEMM).  Reading taken here: "n" on A means A is
# stored [M, K]; "t" on A means A is stored [K, M] and enters as its transpose; "n" on B means B
# is stored [K, N]; "t" on B means B is stored [N, K] and enters as its transpose.  Scales keep
# their logical meaning whatever the storage: one per row of the [M, K] operand and 128-long K
# block, and one per 128x128 (or per row) block of the [N, K] operand; only where the bytes of
# the operands sit changes.

LAYOUTS = ("nt", "nn", "tn", "tt")


def as_mk(a_stored, layout):
    """The [M, K] operand A of D = C + A @ B^T from A as stored under ``layout``."""
    assert layout in LAYOUTS
    return a_stored if layout[0] == "n" else np.asarray(a_stored).T


def as_nk(b_stored, layout):
    """The [N, K] operand B of D = C + A @ B^T from B as stored under ``layout``."""
    assert layout in LAYOUTS
    return b_stored if layout[1] == "t" else np.swapaxes(np.asarray(b_stored), -1, -2)


def gemm_layout(layout, a_stored, sa, b_stored, sb, gran_n=128, c=None, want_abs=False):
    """Dense GEMM under one of the four operand layouts: the NT definition applied to the
    operands read through their storage (``as_mk``, ``as_nk``)."""
    return gemm_nt(as_mk(a_stored, layout), sa, as_nk(b_stored, layout), sb, gran_n, c=c, want_abs=want_abs)


def gemm_layout_points(layout, a_stored, sa, b_stored, sb, ii, jj, gran_n=128, c=None):
    """``gemm_layout`` at output positions (ii[p], jj[p]); returns (D, T)."""
    a = np.ascontiguousarray(as_mk(a_stored, layout))
    b = np.ascontiguousarray(as_nk(b_stored, layout))
    return gemm_nt_points(a, sa, b, sb, ii, jj, gran_n, c=c)


def grouped_contiguous_nn(a_codes, sa, b_stored, sb, grouped_layout, gran_n=128, want_abs=False):
    """M-grouped contiguous GEMM with each group's B stored [K, N] (b_stored [G, K, N])."""
    return grouped_contiguous(a_codes, sa, as_nk(b_stored, "nn"), sb, grouped_layout, gran_n, want_abs=want_abs)


def k_grouped_tn(a_stored, sa, b_stored, sb, ks, c, want_abs=False):
    """K-grouped contiguous GEMM with both operands stored K-outermost: A [sum K, M] and
    B [sum K, N] (the weight-gradient operands as the forward pass leaves them, token-major)."""
    return k_grouped(as_mk(a_stored, "tn"), sa, as_nk(b_stored, "tn"), sb, ks, c, want_abs=want_abs)


def gemm_fp8_fp4_tt(a_stored, sa, b_packed, sb, c=None, want_abs=False):
    """FP8 x FP4 GEMM with A stored [K, M] and the packed FP4 weights stored [N, K/2]."""
    return gemm_fp8_fp4_nt(as_mk(a_stored, "tt"), sa, b_packed, sb, c=c, want_abs=want_abs)
