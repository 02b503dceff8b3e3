"""Number formats used by block-scaled FP8 GEMM, written from their bit definitions.

Test infrastructure only (see the package docstring).

* E4M3 (OCP "E4M3FN", the ``torch.float8_e4m3fn`` format named on page
  "第13章 DeepGEMM" §13.11): sign | 4 exponent bits (bias 7) | 3 mantissa bits,
  subnormals, no infinities, S.1111.111 is NaN, largest finite value 448.
* UE8M0 (page "02 · DeepGEMM 技术解析" §3.1): 8 exponent bits, no sign and no
  mantissa, so every code stands for a power of two, 2^(code - 127); code 0xFF
  is NaN and code 0 (2^-127, the smallest) is the safe padding value.
  Encoding an FP32 scale keeps its exponent field, ``bits >> 23``,
  dropping the mantissa (page "第13章 DeepGEMM" §13.3, second constraint: 0.75
  becomes 0.5 and 3 becomes 2).  The power-of-two test is
  ``(bits & 0x807fffff) == 0`` (page "02 · DeepGEMM 技术解析" §3.1).
* BF16 output: round to nearest, ties to even, computed directly from the
  float64 value (one rounding), with subnormals and overflow to infinity.
* E2M1 (FP4, the weight format of the FP8 x FP4 GEMM on page "第13章 DeepGEMM"
  §13.1 and §13.5; OCP MX "FP4"): sign | 2 exponent bits (bias 1) | 1 mantissa
  bit, a subnormal 0.5, no infinities and no NaN; values 0, 0.5, 1, 1.5, 2, 3,
  4, 6 and their negatives.  Two codes per byte, the lower K index in the low
  nibble.
"""
import numpy as np


def e4m3_decode_table():
    """Return the 256 E4M3 code values as float64 (NaN for 0x7F and 0xFF)."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            v = np.nan
        elif e == 0:
            v = m * 2.0 ** -9              # subnormal: 0.m * 2^(1-7)
        else:
            v = (8 + m) * 2.0 ** (e - 10)  # 1.m * 2^(e-7)
        t[code] = -v if s else v
    return t


_E4M3 = e4m3_decode_table()


def e4m3_decode(codes):
    """Decode an array of E4M3 byte codes (uint8) to float64."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def ue8m0_encode(f32):
    """FP32 scales -> UE8M0 codes by taking the exponent field (uint8)."""
    bits = np.asarray(f32, dtype=np.float32).view(np.uint32)
    return ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.uint8)


def ue8m0_decode(codes):
    """UE8M0 codes -> float64: the power of two 2^(code - 127).

    Code 255 is NaN.  Code 0 is 2^-127: the format has no zero (an FP32 scale of
    0.0 packs to code 0 and so stands for 2^-127).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, (c - 127).astype(np.int32))
    v = np.where(c == 255, np.nan, v)
    return v


def pow2_violation(f32):
    """True where an FP32 scale is not an exact positive-exponent power of two
    (sign or mantissa bits set), i.e. ``(bits & 0x807fffff) != 0``."""
    bits = np.asarray(f32, dtype=np.float32).view(np.uint32)
    return (bits & np.uint32(0x807FFFFF)) != 0


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_rne(x):
    """float64 -> BF16 bit patterns (uint16), one round-to-nearest-even step.

    BF16 has the FP32 exponent range and 8 significand bits.  For |x| in the
    binade [2^e, 2^(e+1)) the spacing is 2^(e-7); below 2^-126 it is the
    subnormal spacing 2^-133.  x / spacing is exact (a power-of-two scaling),
    ``np.rint`` rounds it half-to-even, and the rounded multiple of the
    spacing is exactly representable in FP32, which gives the bits.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    o = out.reshape(-1)
    finite = np.isfinite(flat)
    ax = np.abs(flat)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, e2 = np.frexp(ax)                    # ax = f * 2^e2, f in [0.5, 1)
    e = e2.astype(np.int64) - 1                 # ax in [2^e, 2^(e+1))
    e = np.maximum(e, -126)                     # subnormal spacing below 2^-126
    spacing = np.ldexp(1.0, (e - 7).astype(np.int32))
    r = np.rint(ax / spacing) * spacing
    r = np.where(finite, r, 0.0)
    over = finite & (r > _BF16_MAX)
    r32 = np.where(over, np.inf, r).astype(np.float32)   # exact: r is a BF16 value
    mag = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    sign = np.signbit(flat).astype(np.uint16) << np.uint16(15)
    o[:] = mag | sign
    nan = np.isnan(flat)
    o[nan] = 0x7FC0
    inf = np.isinf(flat)
    o[inf] = np.where(flat[inf] > 0, 0x7F80, 0xFF80).astype(np.uint16)
    return out


def bf16_bits_to_f64(bits):
    """BF16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e2m1_decode_table():
    """Return the 16 E2M1 code values as float64."""
    t = np.empty(16, dtype=np.float64)
    for code in range(16):
        s = (code >> 3) & 1
        e = (code >> 1) & 0x3
        m = code & 0x1
        if e == 0:
            v = m * 0.5                    # subnormal: 0.m * 2^(1-1)
        else:
            v = (2 + m) * 2.0 ** (e - 2)   # 1.m * 2^(e-1)
        t[code] = -v if s else v
    return t


_E2M1 = e2m1_decode_table()


def unpack_fp4(packed, K):
    """Packed FP4 bytes [..., ceil(K/2)] -> codes [..., K] (uint8, 0..15): element 2t is
    the low nibble of byte t, element 2t+1 its high nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    codes[..., 0::2] = p & np.uint8(0x0F)
    codes[..., 1::2] = p >> np.uint8(4)
    return codes[..., :K]


def e2m1_decode(codes):
    """Decode an array of E2M1 codes (0..15) to float64."""
    return _E2M1[np.asarray(codes, dtype=np.uint8) & np.uint8(0x0F)]
