"""Per-token-group FP8 cast: the quantizer whose outputs the GEMM consumes.

Test infrastructure only (see the package docstring).

Recipe (page "02 · DeepGEMM 技术解析" §1.1: activations are cut into 1x128 groups along
K, each group gets one FP32 scale, amax / 448, and is divided by it before the cast to
E4M3; page "第13章 DeepGEMM" §13.3 names the same amax/448 scale):

    s[i, b] = amax_{k in group b} |x[i, k]| / 448      (FP32; s = 1 for an all-zero group)
    q[i, k] = E4M3_RNE(clamp(x[i, k] / s[i, b], -448, 448))

Every step is done in FP32, as the GPU does it, because the quotient decides an integer
code.  For scales stored as UE8M0 (page "02 · DeepGEMM 技术解析" §3.1: powers of two only)
the FP32 scale is raised to the next power of two before the division (reading: rounding
it down, as the layout transform does for a given scale, would push quotients past 448).
The E4M3 rounding here is written as a nearest-value search over the 127 non-negative
finite E4M3 values (ties to the even code), independent of any bit-level encoder.
"""
import numpy as np

from .codecs import e4m3_decode_table

E4M3_MAX = 448.0
GROUP = 128

_T = e4m3_decode_table()
_POS_CODES = np.arange(0x7F, dtype=np.int64)   # 0x00..0x7E: the non-negative finite values
_POS_VALS = _T[_POS_CODES]                       # increasing


def e4m3_encode_rne(x):
    """float32/float64 values in [-448, 448] -> E4M3 codes (uint8), round to nearest with
    ties to the even code.  The sign goes to bit 7 (so -0.0 encodes as 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode_rne takes finite values in [-448, 448]")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    dlo = np.abs(a - _POS_VALS[lo])
    dhi = np.abs(_POS_VALS[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def pow2_ceil(t):
    """Smallest power of two >= t for float32 t >= 0 (1 for t == 0; at least 2^-126), as float32:
    the UE8M0 scale that keeps every quotient of the group within +-448."""
    t = np.asarray(t, dtype=np.float64)
    e = np.ceil(np.log2(np.where(t > 0, t, 1.0)))
    # log2 of a float is not trusted near exact powers: step down while the smaller power still covers t
    p = np.exp2(e)
    p = np.where(p / 2 >= t, p / 2, p)
    p = np.where(p < t, p * 2, p)
    p = np.where(t > 0, np.maximum(p, 2.0 ** -126), 1.0)
    return p.astype(np.float32)


def per_token_group_cast(x, ue8m0=False):
    """x [M, K] (float32 values; K a multiple of 128) -> (codes uint8 [M, K],
    scales float32 [M, K // 128]).  With ue8m0 the scale is amax/448 (FP32) raised to the
    next power of two, so it is exact in UE8M0 and no quotient exceeds 448."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = x.reshape(M, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=2) if M * K else np.zeros((M, K // GROUP), np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    if ue8m0:
        s = pow2_ceil(s)
    q = (g / s[:, :, None]).astype(np.float32)
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode_rne(q.reshape(M, K)), s
