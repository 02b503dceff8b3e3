"""Parity tolerances for block-scaled FP8 GEMM outputs (test code).

FP32 output: |d - o| <= 1e-5 * T + ulp_fp32(o) / 2, where o is the float64
oracle value and T = sum_k |A'_ik B'_jk| over the dequantized operands.  The
half-ulp term is the unavoidable rounding of the output itself; it only
matters where T is tiny next to |C|.

BF16 output: the BF16 result must be within one BF16 ulp of the correctly
rounded oracle value, measured on the ordered integer image of the bit
patterns (this handles binade edges and +-0).  Where |o| is tiny next to T
(cancellation), an FP32-accumulating kernel's own error can exceed one BF16
ulp of o; such an element also passes if |d - o| <= 1e-5 * T + ulp_bf16(d) / 2.
The count of elements that pass only this way is reported.
"""
import numpy as np

from oracle import bf16_rne, bf16_bits_to_f64


def ulp_fp32(x):
    return np.spacing(np.abs(np.asarray(x, dtype=np.float64)).astype(np.float32)).astype(np.float64)


def ulp_bf16(x):
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        _, e2 = np.frexp(ax)
    e = np.maximum(e2.astype(np.int64) - 1, -126)
    return np.ldexp(1.0, (e - 7).astype(np.int32))


def bf16_ordered(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_fp32(d, o, T, rel=1e-5):
    d = np.asarray(d, dtype=np.float64)
    err = np.abs(d - o)
    bound = rel * T + 0.5 * ulp_fp32(o)
    ok = err <= bound
    stats = dict(n=int(ok.size), fail=int((~ok).sum()),
                 max_err_over_T=float(np.max(err / np.maximum(T, 1e-300))) if ok.size else 0.0)
    return ok, stats


def check_bf16(d_bits, o, T, rel=1e-5):
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    r = bf16_rne(o)
    dist = np.abs(bf16_ordered(d_bits) - bf16_ordered(r))
    within_ulp = dist <= 1
    d = bf16_bits_to_f64(d_bits)
    near = np.abs(d - o) <= rel * T + 0.5 * ulp_bf16(d)
    ok = within_ulp | near
    stats = dict(n=int(ok.size), fail=int((~ok).sum()),
                 max_ulp=int(dist.max()) if dist.size else 0,
                 exact=int((dist == 0).sum()),
                 cancellation_only=int((near & ~within_ulp).sum()))
    return ok, stats
