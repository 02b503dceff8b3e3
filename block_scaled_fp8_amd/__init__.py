"""Python binding for libdg.so, the MI355X (gfx950) block-scaled FP8 GEMM library.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  The entry
points follow the library's C ABI (include/dg.h) and the Python API the pages
describe (page "第13章 DeepGEMM" §13.3 and §13.6): ``fp8_gemm_nt((a, sfa), (b, sfb),
d, c=None, recipe=None)`` computes D = C + A @ B.T.

Scale arguments may be given
  * already transformed (path B of page "02 · DeepGEMM 技术解析" §3.2): an
    MN-major tensor, i.e. shape [.., mn, sf_k] (FP32) or [.., mn, ceil(sf_k/4)]
    (int32, packed UE8M0) with strides [.., 1, align4(mn)], as returned by
    ``get_mn_major_tma_aligned_tensor`` / ``..._packed_ue8m0_tensor``; or
  * raw (path A): FP32 [.., mn_blocks, sf_k] contiguous (K-major), in which case the
    library's transform kernel converts them first, on the same stream.
Weight scales for 128x128 blocks (recipe (1, 128, 128)) are passed untransformed,
FP32 [.., ceil(n/128), sf_k] K-major.
"""
import ctypes
import os

import torch

__all__ = [
    "DGError", "lib", "fp8_gemm_nt", "fp8_gemm_nn", "fp8_gemm_tn", "fp8_gemm_tt", "m_grouped_fp8_gemm_nt_contiguous",
    "m_grouped_fp8_gemm_nn_contiguous", "m_grouped_fp8_gemm_nt_masked", "fp8_fp4_gemm_tt",
    "transform_sf", "get_mn_major_tma_aligned_tensor", "get_mn_major_tma_aligned_packed_ue8m0_tensor",
    "per_token_group_cast_fp8", "k_grouped_fp8_gemm_nt_contiguous", "k_grouped_fp8_gemm_tn_contiguous", "transform_sf_into_required_layout",
    "fp8_fp4_gemm_nt", "m_grouped_fp8_fp4_gemm_nt_contiguous", "m_grouped_fp8_fp4_gemm_nt_masked", "get_tma_aligned_size", "get_mk_alignment_for_contiguous_layout", "set_num_sms", "get_num_sms",
    "get_gemm_config", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdg.so")

DG_OUT_BF16, DG_OUT_F32 = 1, 2
DG_SF_F32, DG_SF_UE8M0X4 = 0, 1
DG_IN_BF16, DG_IN_F32 = 1, 2

_i32, _i64, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
_SIGS = {
    **{f"dg_fp8_gemm_{lay}": (_i32, [_i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _i32, _i32,
                                     _p, _i64, _p, _i64, _i32, _p]) for lay in ("nt", "nn", "tn", "tt")},
    "dg_m_grouped_fp8_gemm_nt_contiguous": (_i32, [_i32, _i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _i64,
                                                   _p, _i64, _i64, _i32, _i32, _p, _i64, _i32, _p, _p]),
    "dg_m_grouped_fp8_gemm_nn_contiguous": (_i32, [_i32, _i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _i64,
                                                   _p, _i64, _i64, _i32, _i32, _p, _i64, _i32, _p, _p]),
    "dg_m_grouped_fp8_gemm_nt_masked": (_i32, [_i32, _i32, _i32, _i32, _p, _i64, _i64, _p, _i64, _i64, _p, _i64,
                                               _i64, _p, _i64, _i64, _i32, _i32, _p, _i64, _i64, _i32, _p, _i32, _p]),
    "dg_fp8_fp4_gemm_nt": (_i32, [_i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                                  _i32, _p]),
    "dg_fp8_fp4_gemm_tt": (_i32, [_i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                                  _i32, _p]),
    "dg_m_grouped_fp8_fp4_gemm_nt_contiguous": (_i32, [_i32, _i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _i64,
                                                       _p, _i64, _i64, _p, _i64, _i32, _p, _p]),
    "dg_m_grouped_fp8_fp4_gemm_nt_masked": (_i32, [_i32, _i32, _i32, _i32, _p, _i64, _i64, _p, _i64, _i64, _p, _i64,
                                                   _i64, _p, _i64, _i64, _p, _i64, _i64, _i32, _p, _i32, _p]),
    "dg_transform_sf": (_i32, [_p, _i32, _i32, _i32, _i32, _i32, _p, _p, _p]),
    "dg_k_grouped_fp8_gemm_nt_contiguous": (_i32, [_i32, _i32, _i32, _p, _p, _i64, _p, _p, _i64, _p, _p, _p, _p]),
    "dg_k_grouped_fp8_gemm_tn_contiguous": (_i32, [_i32, _i32, _i32, _p, _p, _i64, _p, _p, _i64, _p, _p, _p, _p]),
    "dg_per_token_group_cast_fp8": (_i32, [_i32, _i32, _p, _i64, _i32, _p, _i64, _p, _i64, _i32, _p]),
    "dg_get_tma_aligned_size": (_i64, [_i64, _i32]),
    "dg_get_mk_alignment_for_contiguous_layout": (_i32, []),
    "dg_set_num_sms": (_i32, [_i32]),
    "dg_get_num_sms": (_i32, []),
    "dg_get_gemm_config": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                  ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                  ctypes.POINTER(_i32)]),
    "dg_get_last_error": (ctypes.c_char_p, []),
}

_lib = None


class DGError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"dg status {status}: {msg}")
        self.status = status


def lib():
    """Load libdg.so (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_scaled_fp8_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status):
    if status != 0:
        raise DGError(status, lib().dg_get_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _a4(x):
    return (int(x) + 3) // 4 * 4


def _codes(t, inner="K"):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"E4M3 operands must be uint8 codes or float8_e4m3fn, got {t.dtype}")
    if t.stride(-1) != 1:
        raise ValueError(f"E4M3 operands must be contiguous along their last dimension ({inner})")
    return t


def _out_dtype(d):
    if d.dtype == torch.bfloat16:
        return DG_OUT_BF16
    if d.dtype == torch.float32:
        return DG_OUT_F32
    raise TypeError(f"output must be bfloat16 or float32, got {d.dtype}")


# ---------------------------------------------------------------- layout helpers
def get_tma_aligned_size(mn, elem_bytes):
    return int(lib().dg_get_tma_aligned_size(int(mn), int(elem_bytes)))


def get_mk_alignment_for_contiguous_layout():
    return int(lib().dg_get_mk_alignment_for_contiguous_layout())


def set_num_sms(n):
    _check(lib().dg_set_num_sms(int(n)))


def get_num_sms():
    return int(lib().dg_get_num_sms())


def get_gemm_config(kind, m, n, k, num_groups=1, expected_m=0, sf_format=DG_SF_F32, gran_n=128,
                    d_dtype=DG_OUT_BF16, num_sms=256):
    """Tile shape the heuristic picks: (block_m, block_n, num_tiles, grid).  Host only."""
    out = [_i32() for _ in range(4)]
    _check(lib().dg_get_gemm_config(kind, m, n, k, num_groups, expected_m, sf_format, gran_n, d_dtype,
                                    num_sms, *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


def transform_sf(sf, mn, gran_mn=1, pack_ue8m0=False, nonpow2_count=None):
    """Raw FP32 scales [(G,) mn_blocks, sf_k] -> MN-major [(G,) mn, sf_k or ceil(sf_k/4)]
    with strides [.., 1, align4(mn)] (FP32, or int32 holding four UE8M0 codes)."""
    if sf.dtype != torch.float32 or not sf.is_contiguous():
        raise ValueError("raw scales must be contiguous float32")
    squeeze = sf.dim() == 2
    sf3 = sf.unsqueeze(0) if squeeze else sf
    G, mnb, sf_k = sf3.shape
    if mnb != (mn + gran_mn - 1) // gran_mn:
        raise ValueError(f"scale rows {mnb} do not match mn={mn} at granularity {gran_mn}")
    a4 = _a4(mn)
    cols = (sf_k + 3) // 4 if pack_ue8m0 else sf_k
    dt = torch.int32 if pack_ue8m0 else torch.float32
    # allocate the whole padded buffer: the kernel writes the padding rows [mn, align4(mn)) too
    flat = torch.empty((G * cols * a4,), dtype=dt, device=sf.device)
    out = flat.as_strided((G, mn, cols), (cols * a4, 1, a4))
    _check(lib().dg_transform_sf(_ptr(sf3), G, mn, sf_k, gran_mn, int(bool(pack_ue8m0)), _ptr(out),
                                 _ptr(nonpow2_count), _stream(sf)))
    return out[0] if squeeze else out


def per_token_group_cast_fp8(x, pack_ue8m0=False, out=None):
    """BF16 or FP32 activations [m, k] (k a multiple of 128) -> (E4M3 codes [m, k] uint8,
    scales MN-major with stride align4(m)), ready for ``fp8_gemm_nt``: FP32 [m, k // 128],
    or with ``pack_ue8m0`` power-of-two scales as int32 [m, ceil(k / 512)] words of four
    UE8M0 codes.  ``out``: an earlier result of the same shape and format to overwrite."""
    if x.dim() != 2 or x.dtype not in (torch.bfloat16, torch.float32) or x.stride(1) != 1:
        raise ValueError("x must be a row-major 2-D bfloat16 or float32 tensor")
    m, k = x.shape
    a4 = _a4(m)
    cols = (k // 128 + 3) // 4 if pack_ue8m0 else k // 128
    if out is not None:
        q, sf = out
        want = torch.int32 if pack_ue8m0 else torch.float32
        if (q.dtype != torch.uint8 or tuple(q.shape) != (m, k) or q.stride(1) != 1 or sf.dtype != want
                or tuple(sf.shape) != (m, cols) or not _is_mn_major(sf)):
            raise ValueError("out must be (uint8 [m, k] codes, MN-major scales) as this call returns them")
    else:
        q = torch.empty((m, k), dtype=torch.uint8, device=x.device)
        flat = torch.empty((max(cols, 1) * a4,), dtype=torch.int32 if pack_ue8m0 else torch.float32, device=x.device)
        sf = flat.as_strided((m, cols), (1, a4))
    _check(lib().dg_per_token_group_cast_fp8(m, k, _ptr(x), x.stride(0), DG_IN_BF16 if x.dtype == torch.bfloat16 else DG_IN_F32,
                                             _ptr(q), q.stride(0), _ptr(sf), a4,
                                             DG_SF_UE8M0X4 if pack_ue8m0 else DG_SF_F32, _stream(x)))
    return q, sf


def transform_sf_into_required_layout(sf, mn, recipe=(1, 128, 128), is_sfa=True, pack_ue8m0=False,
                                      num_groups=None):
    """One entry for both ways of providing scales (page "02 · DeepGEMM 技术解析" §3.2):
    already transformed scales (MN-major FP32, or int32 packed UE8M0 words) are only checked
    and returned; raw FP32 scales ``[(G,) mn_blocks, sf_k]`` are converted on the device.

    ``recipe`` is (gran_m, gran_n, gran_k) with gran_k == 128.  The activation side
    (``is_sfa``) is always per row.  On the weight side gran_n == 128 keeps the 128x128 block
    scales K-major and untransformed (only the LHS scale needs the transposed layout, page
    "第13章 DeepGEMM" §13.3), unless they are to be packed, which broadcasts them per row;
    gran_n == 1 broadcasts raw block scales to every row (or takes per-row scales as they are).
    """
    gran_m, gran_n, gran_k = recipe
    if gran_k != 128 or gran_m != 1 or gran_n not in (1, 128):
        raise ValueError(f"unsupported recipe {recipe}")
    if num_groups is not None and (sf.dim() != 3 or sf.shape[0] != num_groups):
        raise ValueError(f"expected {num_groups} groups of scales, got shape {tuple(sf.shape)}")
    if sf.dtype == torch.int32:
        if not _is_mn_major(sf) or sf.shape[-2] != mn:
            raise ValueError("packed UE8M0 scales must be MN-major [.., mn, ceil(sf_k / 4)]")
        return sf
    if sf.dtype != torch.float32:
        raise TypeError("scales must be float32 or int32 (packed UE8M0)")
    if _is_mn_major(sf) and sf.shape[-2] == mn and sf.shape[-2] > 1:
        if pack_ue8m0:
            raise ValueError("cannot pack already-transformed FP32 scales; pass them raw")
        return sf
    if not is_sfa and gran_n == 128 and not pack_ue8m0:
        if sf.stride(-1) != 1 or sf.shape[-2] != (mn + 127) // 128:
            raise ValueError("128x128 weight scales must be K-major float32 [.., ceil(mn / 128), sf_k]")
        return sf
    gran = 1 if is_sfa else _raw_gran(sf.shape[-2], mn)
    return transform_sf(sf.contiguous(), mn, gran, pack_ue8m0)


def get_mn_major_tma_aligned_tensor(sf):
    return transform_sf(sf.contiguous(), sf.shape[-2], 1, False)


def get_mn_major_tma_aligned_packed_ue8m0_tensor(sf, gran_mn=1, mn=None):
    sf = sf.contiguous()
    mn = sf.shape[-2] * gran_mn if mn is None else mn
    return transform_sf(sf, mn, gran_mn, True)


# ---------------------------------------------------------------- scale marshalling
def _is_mn_major(t):
    """Shape [.., mn, cols] with strides [.., 1, align4(mn)] (the transform's output)."""
    return t.dim() >= 2 and t.stride(-2) == 1 and (t.shape[-2] == 0 or t.stride(-1) == _a4(t.shape[-2]))


def _act_scales(sfa, mn, sf_k, pack):
    """Return (tensor, sf_format) for the activation scales of mn rows (per group)."""
    if sfa.dtype == torch.int32:
        if not _is_mn_major(sfa):
            raise ValueError("packed UE8M0 scales must be MN-major")
        return sfa, DG_SF_UE8M0X4
    if sfa.dtype != torch.float32:
        raise TypeError("scales must be float32 or int32 (packed UE8M0)")
    if _is_mn_major(sfa) and not pack:
        return sfa, DG_SF_F32
    if _is_mn_major(sfa):
        raise ValueError("cannot pack already-transformed FP32 scales; pass them raw")
    t = transform_sf(sfa.contiguous(), mn, 1, pack)
    return t, (DG_SF_UE8M0X4 if pack else DG_SF_F32)


def _weight_scales(sfb, n, sf_k, gran_n, fmt):
    """Return (tensor, stride) for the weight scales of one group."""
    if gran_n == 128:
        if sfb.dtype != torch.float32 or sfb.stride(-1) != 1:
            raise ValueError("128x128 weight scales must be K-major float32 [.., ceil(n/128), sf_k]")
        return sfb, sfb.stride(-2)
    # per-row weight scales, MN-major
    if fmt == DG_SF_UE8M0X4:
        if sfb.dtype == torch.int32:
            return sfb, sfb.stride(-1)
        t = transform_sf(sfb.contiguous(), n, _raw_gran(sfb.shape[-2], n), True)
        return t, t.stride(-1)
    if _is_mn_major(sfb):
        return sfb, sfb.stride(-1)
    t = transform_sf(sfb.contiguous(), n, _raw_gran(sfb.shape[-2], n), False)
    return t, t.stride(-1)


def _raw_gran(rows, n):
    """MN granularity of raw (K-major) weight scales with ``rows`` rows for n weight rows:
    128 when there is one row per 128-row block, else 1.  The two readings coincide only
    for n == 1, where they give the same broadcast."""
    return 128 if rows == (n + 127) // 128 and rows != n else 1


def _recipe_gran_n(recipe, sfa, sfb, n, pack):
    if recipe is not None:
        if tuple(recipe) not in ((1, 128, 128), (1, 1, 128)):
            raise ValueError(f"unsupported recipe {recipe}; use (1, 128, 128) or (1, 1, 128)")
        return recipe[1]
    if sfa.dtype == torch.int32 or pack or sfb.dtype == torch.int32:
        return 1
    if _is_mn_major(sfb) and sfb.shape[-2] == n and n > 1:
        return 1
    return 128


# ---------------------------------------------------------------- GEMMs
def _fp8_gemm(layout, a, b, d, c, recipe, pack_ue8m0):
    """The four operand layouts (page "第13章 DeepGEMM" §13.3): layout[0] "n" = A [M, K], "t" = A
    stored [K, M]; layout[1] "t" = B [N, K], "n" = B stored [K, N].  Scales keep their meaning
    (per row of the [M, K] operand, per block or row of the [N, K] one)."""
    A, sfa = a
    B, sfb = b
    _codes(A, "K" if layout[0] == "n" else "M")
    _codes(B, "K" if layout[1] == "t" else "N")
    M, K = A.shape if layout[0] == "n" else (A.shape[1], A.shape[0])
    N = B.shape[0] if layout[1] == "t" else B.shape[1]
    kb = B.shape[1] if layout[1] == "t" else B.shape[0]
    if kb != K:
        raise ValueError(f"A and B disagree on K ({K} and {kb})")
    sf_k = (K + 127) // 128
    gran_n = _recipe_gran_n(recipe, sfa, sfb, N, pack_ue8m0)
    sfa_t, fmt = _act_scales(sfa, M, sf_k, pack_ue8m0)
    sfb_t, sfb_stride = _weight_scales(sfb, N, sf_k, gran_n, fmt)
    fn = getattr(lib(), "dg_fp8_gemm_" + layout)
    _check(fn(M, N, K, _ptr(A), A.stride(0), _ptr(sfa_t), sfa_t.stride(-1) if M > 0 else 0,
              _ptr(B), B.stride(0), _ptr(sfb_t), sfb_stride, fmt, gran_n,
              _ptr(c), c.stride(0) if c is not None else 0,
              _ptr(d), d.stride(0), _out_dtype(d), _stream(d)))
    return d


def fp8_gemm_nt(a, b, d, c=None, recipe=None, pack_ue8m0=False):
    """D = C + A @ B.T.  ``a = (A [M, K], sfa)``, ``b = (B [N, K], sfb)``, ``d`` [M, N]
    BF16 or FP32 (preallocated); ``c`` optional FP32 [M, N] (may be ``d`` itself)."""
    return _fp8_gemm("nt", a, b, d, c, recipe, pack_ue8m0)


def fp8_gemm_nn(a, b, d, c=None, recipe=None, pack_ue8m0=False):
    """D = C + A @ B with ``a = (A [M, K], sfa)`` and ``b = (B [K, N], sfb)`` (B N-contiguous);
    scales as in ``fp8_gemm_nt``.  K must be at least 256."""
    return _fp8_gemm("nn", a, b, d, c, recipe, pack_ue8m0)


def fp8_gemm_tn(a, b, d, c=None, recipe=None, pack_ue8m0=False):
    """D = C + A.T @ B with ``a = (A [K, M], sfa)`` and ``b = (B [K, N], sfb)`` (both stored
    K-outermost, as token-major activations and gradients are); scales as in ``fp8_gemm_nt``
    (sfa per output row m and 128-long K block).  K must be at least 256."""
    return _fp8_gemm("tn", a, b, d, c, recipe, pack_ue8m0)


def fp8_gemm_tt(a, b, d, c=None, recipe=None, pack_ue8m0=False):
    """D = C + A.T @ B.T with ``a = (A [K, M], sfa)`` and ``b = (B [N, K], sfb)``; scales as in
    ``fp8_gemm_nt``.  K must be at least 256."""
    return _fp8_gemm("tt", a, b, d, c, recipe, pack_ue8m0)


def k_grouped_fp8_gemm_nt_contiguous(a, b, d, ks, c):
    """K-grouped GEMM (MoE weight gradient): ``a = (A [m, sum ks], sfa [sum ks // 128, m])``,
    ``b = (B [n, sum ks], sfb [sum ks // 128, n])`` with FP32 per-row scales, ``ks`` the K of
    each group (multiples of 128), ``d`` and ``c`` FP32 [G, m, n]; ``c`` is required and may be
    ``d`` itself.  D[g] = C[g] + A[:, group g] @ B[:, group g].T (scaled per 128-long block)."""
    return _k_grouped("nt", a, b, d, ks, c)


def k_grouped_fp8_gemm_tn_contiguous(a, b, d, ks, c):
    """As ``k_grouped_fp8_gemm_nt_contiguous`` with both operands stored K-outermost:
    ``a = (A [sum ks, m], sfa)``, ``b = (B [sum ks, n], sfb)`` (the token-major activations and
    gradients of the forward pass); D[g] = C[g] + A[group g].T @ B[group g]."""
    return _k_grouped("tn", a, b, d, ks, c)


def _k_grouped(layout, a, b, d, ks, c):
    A, sfa = a
    B, sfb = b
    _codes(A, "K" if layout == "nt" else "M")
    _codes(B, "K" if layout == "nt" else "N")
    ks = [int(k) for k in ks]
    G = len(ks)
    m, n = (A.shape[0], B.shape[0]) if layout == "nt" else (A.shape[1], B.shape[1])
    if c is None:
        raise ValueError("the K-grouped GEMM requires c (pass d itself to accumulate in place)")
    for t, name in ((sfa, "sfa"), (sfb, "sfb"), (c, "c"), (d, "d")):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor")
    if tuple(d.shape) != (G, m, n) or tuple(c.shape) != (G, m, n):
        raise ValueError(f"c and d must be [{G}, {m}, {n}]")
    if tuple(sfa.shape) != (sum(ks) // 128, m) or tuple(sfb.shape) != (sum(ks) // 128, n):
        raise ValueError("sfa and sfb must be [sum(ks) // 128, m] and [sum(ks) // 128, n]")
    ks_host = (ctypes.c_int32 * G)(*ks)
    fn = getattr(lib(), f"dg_k_grouped_fp8_gemm_{layout}_contiguous")
    _check(fn(G, m, n, ks_host, _ptr(A), A.stride(0), _ptr(sfa), _ptr(B), B.stride(0), _ptr(sfb), _ptr(c), _ptr(d),
              _stream(d)))
    return d


def m_grouped_fp8_gemm_nt_contiguous(a, b, d, grouped_layout, recipe=None, pack_ue8m0=False):
    """Rows of A [sum M_g, K] grouped by ``grouped_layout`` (int32 [sum M_g], -1 = padding);
    ``b = (B [G, N, K], sfb [G, ...])``; D [sum M_g, N]."""
    return _m_grouped_contiguous("nt", a, b, d, grouped_layout, recipe, pack_ue8m0)


def m_grouped_fp8_gemm_nn_contiguous(a, b, d, grouped_layout, recipe=None, pack_ue8m0=False):
    """As ``m_grouped_fp8_gemm_nt_contiguous`` with each group's weights stored [K, N]:
    ``b = (B [G, K, N], sfb [G, ...])`` (page "02 · DeepGEMM 技术解析" §5.1).  K >= 256."""
    return _m_grouped_contiguous("nn", a, b, d, grouped_layout, recipe, pack_ue8m0)


def _m_grouped_contiguous(layout, a, b, d, grouped_layout, recipe, pack_ue8m0):
    A, sfa = a
    B, sfb = b
    _codes(A)
    _codes(B, "K" if layout == "nt" else "N")
    M, K = A.shape
    G, N = B.shape[0], (B.shape[1] if layout == "nt" else B.shape[2])
    if (B.shape[2] if layout == "nt" else B.shape[1]) != K:
        raise ValueError("A and B disagree on K")
    sf_k = (K + 127) // 128
    gran_n = _recipe_gran_n(recipe, sfa, sfb, N, pack_ue8m0)
    sfa_t, fmt = _act_scales(sfa, M, sf_k, pack_ue8m0)
    sfb_t, sfb_stride = _weight_scales(sfb, N, sf_k, gran_n, fmt)
    if grouped_layout.dtype != torch.int32 or not grouped_layout.is_contiguous():
        raise ValueError("grouped_layout must be contiguous int32")
    fn = getattr(lib(), f"dg_m_grouped_fp8_gemm_{layout}_contiguous")
    _check(fn(
        M, N, K, G, _ptr(A), A.stride(0), _ptr(sfa_t), sfa_t.stride(-1), _ptr(B), B.stride(1), B.stride(0),
        _ptr(sfb_t), sfb_stride, sfb_t.stride(0), fmt, gran_n, _ptr(d), d.stride(0), _out_dtype(d),
        _ptr(grouped_layout), _stream(d)))
    return d


def m_grouped_fp8_gemm_nt_masked(a, b, d, masked_m, expected_m=0, recipe=None, pack_ue8m0=False):
    """A [G, M_max, K] with ``masked_m`` (int32 [G], device) valid rows per group;
    ``b = (B [G, N, K], sfb [G, ...])``; D [G, M_max, N] (rows past masked_m untouched)."""
    A, sfa = a
    B, sfb = b
    _codes(A)
    _codes(B)
    G, Mmax, K = A.shape
    N = B.shape[1]
    sf_k = (K + 127) // 128
    gran_n = _recipe_gran_n(recipe, sfa, sfb, N, pack_ue8m0)
    sfa_t, fmt = _act_scales(sfa, Mmax, sf_k, pack_ue8m0)
    sfb_t, sfb_stride = _weight_scales(sfb, N, sf_k, gran_n, fmt)
    if masked_m.dtype != torch.int32 or not masked_m.is_contiguous():
        raise ValueError("masked_m must be contiguous int32")
    _check(lib().dg_m_grouped_fp8_gemm_nt_masked(
        G, Mmax, N, K, _ptr(A), A.stride(1), A.stride(0), _ptr(sfa_t), sfa_t.stride(-1), sfa_t.stride(0),
        _ptr(B), B.stride(1), B.stride(0), _ptr(sfb_t), sfb_stride, sfb_t.stride(0), fmt, gran_n,
        _ptr(d), d.stride(1), d.stride(0), _out_dtype(d), _ptr(masked_m), int(expected_m), _stream(d)))
    return d


# ---------------------------------------------------------------- FP8 activations x FP4 weights
def _fp4_codes(t, k):
    """Packed E2M1 weights: uint8 (or float4_e2m1fn_x2) [.., n, k // 2], K-contiguous."""
    if t.dtype != torch.uint8 and str(t.dtype) != "torch.float4_e2m1fn_x2":
        raise TypeError(f"FP4 weights must be uint8 bytes or float4_e2m1fn_x2 (two codes per byte), got {t.dtype}")
    if t.stride(-1) != 1 or t.shape[-1] != k // 2:
        raise ValueError(f"FP4 weights must be K-contiguous [.., n, k // 2] = [.., n, {k // 2}]")
    return t


def _fp4_act_scales(sfa, m):
    """Activation scales of the FP8 x FP4 GEMM: packed UE8M0 words (MN-major), or raw FP32
    power-of-two scales [.., m, k // 128] which the transform packs."""
    if sfa.dtype == torch.int32:
        if not _is_mn_major(sfa):
            raise ValueError("packed UE8M0 scales must be MN-major")
        return sfa
    if sfa.dtype != torch.float32:
        raise TypeError("scales must be float32 (powers of two) or int32 (packed UE8M0)")
    return transform_sf(sfa.contiguous(), m, 1, True)


def _fp4_weight_scales(sfb, n, k):
    """Weight scales of FP4 weights, one per row and 32 K: int32 words [.., n, k // 128]
    (MN-major, stride align4(n)), or raw FP32 [.., n, k // 32] which the transform packs
    four 32-K codes per word."""
    if sfb.dtype == torch.int32:
        if not _is_mn_major(sfb) or sfb.shape[-1] != k // 128:
            raise ValueError("packed FP4 weight scales must be MN-major int32 [.., n, k // 128]")
        return sfb
    if sfb.dtype != torch.float32 or sfb.shape[-1] != k // 32 or sfb.shape[-2] != n:
        raise ValueError(f"raw FP4 weight scales must be float32 [.., {n}, {k // 32}]")
    return transform_sf(sfb.contiguous(), n, 1, True)


def fp8_fp4_gemm_nt(a, b, d, c=None):
    """D = C + A @ B.T with FP8 activations and FP4 weights.  ``a = (A [M, K] E4M3, sfa)``,
    sfa one power-of-two scale per row and 128 K; ``b = (B [N, K // 2] packed E2M1, sfb)``,
    sfb one power-of-two scale per row and 32 K; ``d`` [M, N] BF16 or FP32; ``c`` optional FP32."""
    return _fp8_fp4_gemm("nt", a, b, d, c)


def fp8_fp4_gemm_tt(a, b, d, c=None):
    """As ``fp8_fp4_gemm_nt`` with the activations stored [K, M] (``a = (A [K, M], sfa)``)."""
    return _fp8_fp4_gemm("tt", a, b, d, c)


def _fp8_fp4_gemm(layout, a, b, d, c):
    A, sfa = a
    B, sfb = b
    _codes(A, "K" if layout == "nt" else "M")
    M, K = A.shape if layout == "nt" else (A.shape[1], A.shape[0])
    _fp4_codes(B, K)
    N = B.shape[0]
    sfa_t = _fp4_act_scales(sfa, M)
    sfb_t = _fp4_weight_scales(sfb, N, K)
    _check(getattr(lib(), "dg_fp8_fp4_gemm_" + layout)(M, N, K, _ptr(A), A.stride(0), _ptr(sfa_t), sfa_t.stride(-1) if M > 0 else 0,
                                    _ptr(B), B.stride(0), _ptr(sfb_t), sfb_t.stride(-1) if N > 0 else 0,
                                    _ptr(c), c.stride(0) if c is not None else 0,
                                    _ptr(d), d.stride(0), _out_dtype(d), _stream(d)))
    return d


def m_grouped_fp8_fp4_gemm_nt_contiguous(a, b, d, grouped_layout):
    """Rows of A [sum M_g, K] grouped by ``grouped_layout``; ``b = (B [G, N, K // 2] packed E2M1,
    sfb [G, N, ..])``; D [sum M_g, N] BF16."""
    A, sfa = a
    B, sfb = b
    _codes(A)
    M, K = A.shape
    _fp4_codes(B, K)
    G, N, _ = B.shape
    sfa_t = _fp4_act_scales(sfa, M)
    sfb_t = _fp4_weight_scales(sfb, N, K)
    if grouped_layout.dtype != torch.int32 or not grouped_layout.is_contiguous():
        raise ValueError("grouped_layout must be contiguous int32")
    _check(lib().dg_m_grouped_fp8_fp4_gemm_nt_contiguous(
        M, N, K, G, _ptr(A), A.stride(0), _ptr(sfa_t), sfa_t.stride(-1), _ptr(B), B.stride(1), B.stride(0),
        _ptr(sfb_t), sfb_t.stride(-1), sfb_t.stride(0), _ptr(d), d.stride(0), _out_dtype(d),
        _ptr(grouped_layout), _stream(d)))
    return d


def m_grouped_fp8_fp4_gemm_nt_masked(a, b, d, masked_m, expected_m=0):
    """A [G, M_max, K] with ``masked_m`` valid rows per group; ``b = (B [G, N, K // 2] packed E2M1,
    sfb [G, N, ..])``; D [G, M_max, N] BF16 (rows past masked_m untouched)."""
    A, sfa = a
    B, sfb = b
    _codes(A)
    G, Mmax, K = A.shape
    _fp4_codes(B, K)
    N = B.shape[1]
    sfa_t = _fp4_act_scales(sfa, Mmax)
    sfb_t = _fp4_weight_scales(sfb, N, K)
    if masked_m.dtype != torch.int32 or not masked_m.is_contiguous():
        raise ValueError("masked_m must be contiguous int32")
    _check(lib().dg_m_grouped_fp8_fp4_gemm_nt_masked(
        G, Mmax, N, K, _ptr(A), A.stride(1), A.stride(0), _ptr(sfa_t), sfa_t.stride(-1), sfa_t.stride(0),
        _ptr(B), B.stride(1), B.stride(0), _ptr(sfb_t), sfb_t.stride(-1), sfb_t.stride(0),
        _ptr(d), d.stride(1), d.stride(0), _out_dtype(d), _ptr(masked_m), int(expected_m), _stream(d)))
    return d
