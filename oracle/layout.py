"""Reference for the scale-layout transform.  Test infrastructure only.

Page "02 · DeepGEMM 技术解析" §3.1 (scale tensor contract) and §3.2 (the two
ways of providing scales, recipe broadcast along MN); page "第13章 DeepGEMM"
§13.3 (the LHS scale must be transposed and aligned; packing keeps the
exponent field).

Input: FP32 scales ``sf[g, mn_block, kb]`` (K-major, contiguous), where
``mn_block = r // gran_mn`` for row ``r`` (``gran_mn`` is 1, or 128 when a
128x128 weight-block scale is broadcast to every row of its block).

Output, FP32 mode: a flat buffer per group holding element ``(r, kb)`` at
``kb * align4(mn) + r`` (MN-major, each K slice padded to a multiple of four
entries = 16 bytes).  Packed mode: int32 words, word ``(r, q)`` at
``q * align4(mn) + r``, whose byte ``t`` (bits 8t..8t+7) is the UE8M0 code of
K-block ``4q + t`` -- four consecutive K positions, little-endian by K index.
Padding rows ``mn <= r < align4(mn)`` and tail bytes ``4q + t >= sf_k`` are 0
(the pages say padding is never read; zero is the safe finite code).
"""
import numpy as np

from .codecs import ue8m0_encode, ue8m0_decode, pow2_violation


def align4(x):
    return (int(x) + 3) // 4 * 4


def transform_sf(sf, mn, gran_mn=1, pack_ue8m0=False):
    """Return (out, nonpow2_count).

    ``sf``: float32 array [G, mn_blocks, sf_k] or [mn_blocks, sf_k].
    ``out``: float32 [G, sf_k, align4(mn)] or int32 [G, ceil(sf_k/4), align4(mn)]
    (the leading G axis dropped when the input had none).
    ``nonpow2_count``: number of input scales failing the power-of-two mask
    (only counted when packing).
    """
    sf = np.asarray(sf, dtype=np.float32)
    squeeze = sf.ndim == 2
    if squeeze:
        sf = sf[None]
    G, mnb, sf_k = sf.shape
    assert mnb == (mn + gran_mn - 1) // gran_mn, "mn_blocks does not match mn / gran_mn"
    a4 = align4(mn)
    count = 0
    rows = np.arange(mn) // gran_mn                    # scale block of each row
    per_row = sf[:, rows, :]                           # [G, mn, sf_k]
    if not pack_ue8m0:
        out = np.zeros((G, sf_k, a4), dtype=np.float32)
        out[:, :, :mn] = per_row.transpose(0, 2, 1)
    else:
        pk = (sf_k + 3) // 4
        codes = np.zeros((G, mn, 4 * pk), dtype=np.uint32)   # tail K slots stay 0
        codes[:, :, :sf_k] = ue8m0_encode(per_row)
        count = int(pow2_violation(sf).sum())
        words = np.zeros((G, mn, pk), dtype=np.uint32)
        for t in range(4):                             # byte t <- K-block 4q + t
            words |= codes[:, :, t::4] << np.uint32(8 * t)
        out = np.zeros((G, pk, a4), dtype=np.uint32)
        out[:, :, :mn] = words.transpose(0, 2, 1)
        out = out.view(np.int32)
    if squeeze:
        out = out[0]
    return out, count


def unpack_ue8m0(packed, mn, sf_k):
    """Packed int32 [.., ceil(sf_k/4), align4(mn)] -> float64 scales [.., mn, sf_k]."""
    p = np.asarray(packed).view(np.uint32)
    squeeze = p.ndim == 2
    if squeeze:
        p = p[None]
    G = p.shape[0]
    out = np.empty((G, mn, sf_k), dtype=np.float64)
    for kb in range(sf_k):
        q, t = divmod(kb, 4)
        codes = ((p[:, q, :mn] >> np.uint32(8 * t)) & np.uint32(0xFF)).astype(np.uint8)
        out[:, :, kb] = ue8m0_decode(codes)
    return out[0] if squeeze else out
