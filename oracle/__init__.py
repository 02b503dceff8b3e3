"""Float64 CPU oracle for fine-grained block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (``block_scaled_fp8_amd``) and imports nothing from it.

What it computes (page "02 · DeepGEMM 技术解析", §1.1 and §2.2; page "第13章
DeepGEMM", §13.3 algorithm and "点 1"; page "LinearQaunt-分块量化矩阵乘法",
the dequantize-then-matmul description):

    D[i, j] = C[i, j] + sum_b  sa[i, b] * sb[beta(j), b] * P[i, j, b]
    P[i, j, b] = sum_{k in K-block b} dec(A[i, k]) * dec(B[j, k])

with 128-long K blocks, beta(j) = j // 128 for 128x128 weight blocks and
beta(j) = j for per-row weight scales.  Every finite E4M3 value is a multiple
of 2^-9 with magnitude <= 448, so each block partial P is an exact float64
number whatever order it is summed in; only the scale products and the sum
over blocks round (one float64 rounding each).

Modules:
  codecs  -- E4M3 and E2M1 decode, FP4 unpacking, UE8M0 encode/decode,
             float64 -> BF16 round-to-nearest-even
  layout  -- the scale-layout transform (MN-major, 4-aligned stride, UE8M0 x4 packing)
  gemm    -- dense NT, M-grouped contiguous, M-grouped masked and K-grouped references,
             the FP8 x FP4 GEMM (E2M1 weights with one scale per 32 K) in the dense and
             M-grouped forms, and the nn / tn / tt operand layouts (operands stored
             transposed)
  quant   -- the per-token-group FP8 cast (E4M3 codes and 1x128 FP32 scales)

Parity pins: every function here is pinned by a `-m "not gpu"` test in
``tests/test_oracle_pins.py`` against something other than itself (closed
forms, worked examples printed on the pages, exact rational brute force,
library routines on special cases).  No function is "parity unpinned"; the
comparison with the original CUDA library itself cannot be made here.
"""
from . import codecs, layout, gemm, quant  # noqa: F401
from .codecs import (e4m3_decode_table, e4m3_decode, ue8m0_encode, ue8m0_decode,
                     bf16_rne, bf16_bits_to_f64, pow2_violation, e2m1_decode_table, e2m1_decode,
                     unpack_fp4)  # noqa: F401
from .layout import align4, transform_sf, unpack_ue8m0  # noqa: F401
from .gemm import (gemm_nt, gemm_nt_points, grouped_contiguous, grouped_masked, k_grouped,
                   expand_scales_b, gemm_fp8_fp4_nt, gemm_fp8_fp4_nt_points, grouped_contiguous_fp8_fp4,
                   grouped_masked_fp8_fp4, LAYOUTS, as_mk, as_nk, gemm_layout, gemm_layout_points,
                   grouped_contiguous_nn, k_grouped_tn, gemm_fp8_fp4_tt)  # noqa: F401
from .quant import e4m3_encode_rne, per_token_group_cast  # noqa: F401
