/*
 * dg.h -- C ABI of the MI355X (gfx950) block-scaled FP8 GEMM library (libdg.so).
 *
 * The library computes the fine-grained block-scaled FP8 GEMM
 *
 *     D = C + A . B^T
 *
 * where A holds OCP E4M3 activations with one scale per 1x128 group along K
 * and B holds E4M3 weights with one scale per 128x128 block (or one per row
 * and 128 K values).  K is consumed in 128-long blocks; each block's partial
 * product is promoted into an FP32 accumulator as
 *     final += scale_a * scale_b * partial
 * Definitions: page "02 · DeepGEMM 技术解析" (PaperTrace) §1.1 (the
 * quantisation recipe), §2.2 (two-level accumulation), §2.3 (1-D / 2-D weight
 * scales), §3.1-3.2 (scale layouts and the two ways of providing them), §5.1-5.2
 * (M-grouped contiguous and masked layouts); page "第13章 DeepGEMM：FP4 / FP8
 * 矩阵乘法内核" §13.3 (interface D = C + A @ B.T, the "nt" naming, the
 * algorithm box) and §13.6 (M-grouped GEMM).
 *
 * Conventions for every entry point
 *  - Every data pointer is DEVICE memory owned and allocated by the caller.
 *    The library allocates nothing and keeps no per-call state; the only
 *    global is the persistent grid size (dg_set_num_sms).
 *  - Strides are in ELEMENTS of the pointed-to type.  "E4M3" buffers are
 *    bytes (uint8 codes), "F32" are float, "UE8M0x4" are int32 words each
 *    holding four UE8M0 codes (byte t = K-block 4q+t, little-endian by K).
 *  - sf_k = ceil(k / 128); packed_sf_k = ceil(sf_k / 4); align4(x) = 4*ceil(x/4).
 *  - Every call is enqueued on `stream` and returns without synchronising.
 *  - Arguments are validated on the host before any HIP call.  A bad argument
 *    returns a negative dg_status and leaves a message for dg_get_last_error();
 *    nothing is launched.  A failed launch returns DG_ERR_HIP.  Nothing aborts.
 *  - Device-side anomalies are skipped, never trapped: rows whose group index
 *    is negative or >= num_groups produce no output.
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_NULL = -1,        /* a required pointer is NULL */
  DG_ERR_DTYPE = -2,       /* unknown output dtype or scale format */
  DG_ERR_SHAPE = -3,       /* sizes out of range or inconsistent */
  DG_ERR_LAYOUT = -4,      /* strides / alignment do not match the contract */
  DG_ERR_UNSUPPORTED = -5, /* a valid but unsupported combination (e.g. C with BF16 D) */
  DG_ERR_HIP = -6          /* a HIP runtime call or launch failed */
} dg_status;

typedef enum { DG_OUT_BF16 = 1, DG_OUT_F32 = 2 } dg_out_dtype;
typedef enum { DG_SF_F32 = 0, DG_SF_UE8M0X4 = 1 } dg_sf_format;
typedef enum { DG_IN_BF16 = 1, DG_IN_F32 = 2 } dg_in_dtype;

/*
 * Dense NT GEMM: D[m, n] = C[m, n] + sum_b sa[m, b] * sb[.., b] * sum_{k in block b} A[m, k] * B[n, k]
 * (page "第13章 DeepGEMM" §13.3: fp8_gemm_nt computes D = C + A @ B.T).
 *
 *  m, n, k      : problem sizes; k > 0 and k % 128 == 0; m, n >= 0.  m == 0 or n == 0 is a
 *                 no-op that reads and writes nothing (its pointers may then be NULL).
 *  a, lda       : A E4M3 [m, k], element (i, kk) at a[i*lda + kk]; k <= lda < 2^23, lda % 16 == 0,
 *                 a 16-byte aligned.
 *  sfa, sfa_stride : activation scales, MN-major (the LHS scale must be transposed and
 *                 aligned, page "第13章 DeepGEMM" §13.3 constraint 1; layout page
 *                 "02 · DeepGEMM 技术解析" §3.1).  F32: element (i, b) at sfa[b*sfa_stride + i];
 *                 UE8M0x4: word (i, q) at sfa[q*sfa_stride + i].  sfa_stride == align4(m).
 *  b, ldb       : B E4M3 [n, k], element (j, kk) at b[j*ldb + kk]; same rules as A.
 *  sfb, sfb_stride : weight scales.
 *                 gran_n == 128 (128x128 blocks, "1d2d"): F32 only, K-major [ceil(n/128), sf_k],
 *                   element (jb, b) at sfb[jb*sfb_stride + b]; sfb_stride >= sf_k.  Only the
 *                   LHS scale needs transposing (§13.3 constraint 1).
 *                 gran_n == 1 (one scale per weight row, "1d1d"; path B of §3.2 broadcasts the
 *                   128x128 block scale to every row): MN-major like sfa, stride == align4(n).
 *  sf_format    : DG_SF_F32 or DG_SF_UE8M0X4 (applies to both sfa and sfb; UE8M0x4 requires
 *                 gran_n == 1).
 *  c, ldc       : NULL, or FP32 [m, n] at c[i*ldc + j] (requires d_dtype == DG_OUT_F32),
 *                 ldc >= n, 4-byte aligned.  c may alias d (then ldc must equal ldd): D
 *                 accumulates in place.
 *  d, ldd, d_dtype : output [m, n] at d[i*ldd + j], BF16 (round to nearest even) or FP32;
 *                 ldd >= n, d aligned to its element size.  Rows are written with 4-element
 *                 vector stores when ldd % 4 == 0 and d is 16-byte aligned, element stores
 *                 otherwise.
 * Returns DG_OK or a negative dg_status.
 */
int dg_fp8_gemm_nt(int32_t m, int32_t n, int32_t k,
                   const void* a, int64_t lda,
                   const void* sfa, int64_t sfa_stride,
                   const void* b, int64_t ldb,
                   const void* sfb, int64_t sfb_stride,
                   int32_t sf_format, int32_t gran_n,
                   const float* c, int64_t ldc,
                   void* d, int64_t ldd, int32_t d_dtype,
                   hipStream_t stream);

/*
 * The other three operand layouts (page "第13章 DeepGEMM" §13.3: D = C + A @ B, the suffix
 * letters giving the transposition of A and of B; fp8_gemm_nn / tn / tt).  Same arguments and
 * the same D as dg_fp8_gemm_nt except where A or B sits in memory:
 *  - "t" on A (dg_fp8_gemm_tn, dg_fp8_gemm_tt): A stored [k, m], element (i, kk) at
 *    a[kk*lda + i]; m <= lda < 2^23, lda % 16 == 0, k * lda < 2^31, a 16-byte aligned.
 *  - "n" on B (dg_fp8_gemm_nn, dg_fp8_gemm_tn): B stored [k, n], element (j, kk) at
 *    b[kk*ldb + j]; n <= ldb < 2^23, ldb % 16 == 0, k * ldb < 2^31, b 16-byte aligned.
 * Scales keep their meaning and layout: sfa per row i of D and 128-long K block, sfb per
 * 128x128 block (FP32) or per row j of D (packed UE8M0 only: per-row FP32 weight scales return
 * DG_ERR_UNSUPPORTED here).  k >= 256 (DG_ERR_UNSUPPORTED below).  The operands stored
 * [k, x] are staged in LDS (as 32-column strips, or as whole K rows with an XOR key per row
 * when the tile side is 128 or 256 wide) and fed to the matrix unit with the transposing LDS
 * read, so no transposed copy is made and no workspace is used.
 */
int dg_fp8_gemm_nn(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                   const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride, int32_t sf_format, int32_t gran_n,
                   const float* c, int64_t ldc, void* d, int64_t ldd, int32_t d_dtype, hipStream_t stream);
int dg_fp8_gemm_tn(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                   const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride, int32_t sf_format, int32_t gran_n,
                   const float* c, int64_t ldc, void* d, int64_t ldd, int32_t d_dtype, hipStream_t stream);
int dg_fp8_gemm_tt(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                   const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride, int32_t sf_format, int32_t gran_n,
                   const float* c, int64_t ldc, void* d, int64_t ldd, int32_t d_dtype, hipStream_t stream);

/*
 * M-grouped contiguous GEMM (page "02 · DeepGEMM 技术解析" §5.1; page "第13章 DeepGEMM"
 * §13.6): the rows of A are the concatenated tokens of num_groups experts; row i uses
 * expert g = grouped_layout[i], i.e. D[i, :] = A[i, :] . B[g]^T with g's scales.  Only M is
 * grouped: N and K are the same for every group.
 *
 *  m_total      : rows of A and D (sum of the group segments, including padding rows).
 *  grouped_layout : device int32 [m_total], the group of each row; a negative value marks a
 *                 padding row whose D row is not written.  Precondition (not checked, it would
 *                 need a device read): every aligned block of
 *                 dg_get_mk_alignment_for_contiguous_layout() rows belongs to one group, padding
 *                 rows of a block come after its group's rows, and the group of a block is read
 *                 from its first row (a block whose first row is negative is skipped).
 *  b, b_group_stride : B [num_groups, n, k]; group g starts at b + g*b_group_stride.
 *  sfb_group_stride  : group g's weight scales start at sfb + g*sfb_group_stride.
 *  Other arguments as in dg_fp8_gemm_nt (sfa covers all m_total rows, stride align4(m_total)).
 *  No C term (BF16 or FP32 D).
 */
int dg_m_grouped_fp8_gemm_nt_contiguous(int32_t m_total, int32_t n, int32_t k, int32_t num_groups,
                                        const void* a, int64_t lda,
                                        const void* sfa, int64_t sfa_stride,
                                        const void* b, int64_t ldb, int64_t b_group_stride,
                                        const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                        int32_t sf_format, int32_t gran_n,
                                        void* d, int64_t ldd, int32_t d_dtype,
                                        const int32_t* grouped_layout,
                                        hipStream_t stream);

/*
 * M-grouped contiguous GEMM with each group's weights stored [k, n] (page "02 · DeepGEMM
 * 技术解析" §5.1 names m_grouped_fp8_gemm_{nt, nn}_contiguous): element (j, kk) of group g at
 * b[g*b_group_stride + kk*ldb + j], n <= ldb < 2^23, ldb % 16 == 0, k * ldb < 2^31,
 * b_group_stride >= k*ldb.  Everything else as in dg_m_grouped_fp8_gemm_nt_contiguous;
 * k >= 256, 128x128 FP32 or per-row UE8M0 weight scales.
 */
int dg_m_grouped_fp8_gemm_nn_contiguous(int32_t m_total, int32_t n, int32_t k, int32_t num_groups,
                                        const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                                        const void* b, int64_t ldb, int64_t b_group_stride,
                                        const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                        int32_t sf_format, int32_t gran_n, void* d, int64_t ldd, int32_t d_dtype,
                                        const int32_t* grouped_layout, hipStream_t stream);

/*
 * M-grouped masked GEMM (page "02 · DeepGEMM 技术解析" §5.2): A is [num_groups, m_max, k]
 * with a static shape (so the call can sit in a captured graph); group g has
 * masked_m[g] valid rows, read on the device.  Only rows i < clamp(masked_m[g], 0, m_max)
 * are computed and written; the other rows of D are left untouched.
 *
 *  a, lda, a_group_stride : row i of group g at a + g*a_group_stride + i*lda.
 *  sfa, sfa_stride, sfa_group_stride : group g's activation scales (MN-major over m_max rows,
 *                 sfa_stride == align4(m_max)) start at sfa + g*sfa_group_stride.
 *  b, ..., sfb_group_stride : as in the contiguous variant.
 *  d, ldd, d_group_stride : row i of group g at d + g*d_group_stride + i*ldd.
 *  masked_m     : device int32 [num_groups].
 *  expected_m   : host hint (typical valid rows per group) used only to choose the tile
 *                 shape; it never changes which rows are computed.  <= 0 means m_max.
 */
int dg_m_grouped_fp8_gemm_nt_masked(int32_t num_groups, int32_t m_max, int32_t n, int32_t k,
                                    const void* a, int64_t lda, int64_t a_group_stride,
                                    const void* sfa, int64_t sfa_stride, int64_t sfa_group_stride,
                                    const void* b, int64_t ldb, int64_t b_group_stride,
                                    const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                    int32_t sf_format, int32_t gran_n,
                                    void* d, int64_t ldd, int64_t d_group_stride, int32_t d_dtype,
                                    const int32_t* masked_m, int32_t expected_m,
                                    hipStream_t stream);

/*
 * FP8 activations x FP4 weights (page "第13章 DeepGEMM" §13.1: the V4 routed-expert recipe,
 * FP8 activations and FP4 weights with one weight scale per 32 K elements; §13.5: the FP4
 * weights go into the MMA next to the FP8 activations and the power-of-two scales are applied
 * inside it; page "02 · DeepGEMM 技术解析" §3.1: UE8M0 scales packed four per int32):
 *
 *   D[i, j] = C[i, j] + sum_b sa[i, b] * sum_{t=0..3} sb[j, 4b+t] * sum_{k in K [128b+32t, +32)} A[i, k] * B[j, k]
 *
 *  m, n, k      : k % 128 == 0 and k >= 256 (two K blocks; DG_ERR_UNSUPPORTED below); m, n >= 0
 *                 (m == 0 or n == 0 is a no-op).
 *  a, lda       : A E4M3 [m, k] as in dg_fp8_gemm_nt.
 *  sfa, sfa_stride : UE8M0 activation scales, one per row and 128-long K block, packed four per
 *                 int32 and MN-major exactly as dg_fp8_gemm_nt's DG_SF_UE8M0X4 sfa
 *                 (word (i, q) at sfa[q*sfa_stride + i], byte t = K block 4q+t); sfa_stride == align4(m).
 *  b, ldb       : B E2M1 (FP4: 1 sign, 2 exponent, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6
 *                 and their negatives) [n, k], two codes per byte: element (j, kk) is the low nibble
 *                 of byte b[j*ldb + kk/2] for even kk and its high nibble for odd kk.  ldb (BYTES)
 *                 >= k/2, ldb % 16 == 0, < 2^23; b 16-byte aligned.
 *  sfb, sfb_stride : UE8M0 weight scales, one per row and 32-long K group: int32 word (j, b) at
 *                 sfb[b*sfb_stride + j] holds row j's four codes of K block b, byte t for K
 *                 [128b + 32t, +32) (dg_transform_sf with sf_k = k/32 and pack_ue8m0 = 1 produces
 *                 this layout from FP32 per-32 scales); sfb_stride == align4(n).  16-byte aligned.
 *                 A code c stands for 2^(c - 127).
 *  c, ldc, d, ldd, d_dtype : as in dg_fp8_gemm_nt (C only with FP32 D; C may alias D).
 * Returns DG_OK or a negative dg_status.
 */
int dg_fp8_fp4_gemm_nt(int32_t m, int32_t n, int32_t k,
                       const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                       const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                       const float* c, int64_t ldc,
                       void* d, int64_t ldd, int32_t d_dtype,
                       hipStream_t stream);

/*
 * FP8 x FP4 GEMM with the activations stored [k, m] (page "第13章 DeepGEMM" §13.3 and §13.5:
 * fp8_fp4_gemm_{nt,nn,tn,tt}; the FP4 weights stay [n, k/2], K-packed): element (i, kk) of A
 * at a[kk*lda + i], m <= lda < 2^23, lda % 16 == 0, k * lda < 2^31.  Everything else as in
 * dg_fp8_fp4_gemm_nt.  (Weights stored [k, n] would pack two N values per byte; that form is
 * not provided.)
 */
int dg_fp8_fp4_gemm_tt(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                       int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                       const float* c, int64_t ldc, void* d, int64_t ldd, int32_t d_dtype, hipStream_t stream);

/*
 * M-grouped contiguous FP8 x FP4 GEMM (page "第13章 DeepGEMM" §13.6, the MoE prefill form with
 * FP4 expert weights): rows grouped as in dg_m_grouped_fp8_gemm_nt_contiguous; operands and
 * scales as in dg_fp8_fp4_gemm_nt; group g's packed weights start at b + g*b_group_stride
 * (bytes) and its scale words at sfb + g*sfb_group_stride (>= (k/128)*sfb_stride).  BF16 D only.
 */
int dg_m_grouped_fp8_fp4_gemm_nt_contiguous(int32_t m_total, int32_t n, int32_t k, int32_t num_groups,
                                            const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                                            const void* b, int64_t ldb, int64_t b_group_stride,
                                            const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                            void* d, int64_t ldd, int32_t d_dtype,
                                            const int32_t* grouped_layout, hipStream_t stream);

/*
 * M-grouped masked FP8 x FP4 GEMM (page "02 · DeepGEMM 技术解析" §5.2; page "第13章 DeepGEMM"
 * §13.6, the decode form): groups and masked_m as in dg_m_grouped_fp8_gemm_nt_masked;
 * operands and scales as in dg_fp8_fp4_gemm_nt, per group (sfa_group_stride >=
 * ceil(k/512)*sfa_stride, sfb_group_stride >= (k/128)*sfb_stride).  BF16 D only.
 */
int dg_m_grouped_fp8_fp4_gemm_nt_masked(int32_t num_groups, int32_t m_max, int32_t n, int32_t k,
                                        const void* a, int64_t lda, int64_t a_group_stride,
                                        const void* sfa, int64_t sfa_stride, int64_t sfa_group_stride,
                                        const void* b, int64_t ldb, int64_t b_group_stride,
                                        const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                        void* d, int64_t ldd, int64_t d_group_stride, int32_t d_dtype,
                                        const int32_t* masked_m, int32_t expected_m,
                                        hipStream_t stream);

/*
 * K-grouped contiguous GEMM, the MoE weight-gradient form (page "02 · DeepGEMM 技术解析" §3.3:
 * groups concatenated along K, two-dimensional [sum_sf_k, mn] FP32 scales, mn % 4 == 0, C
 * required and best passed as D itself; page "第13章 DeepGEMM" §13.6 and §13.13: M and N
 * fixed, the groups split K):
 *
 *   D[g] = C[g] + sum_{b in group g's K blocks} sa[b, i] * sb[b, j] * sum_{k in block b} A[i, k] * B[j, k]
 *
 *  num_groups   : > 0.  ks: HOST int32 [num_groups], group g's K (a multiple of 128, 0 allowed:
 *                 then D[g] = C[g]); group g covers K columns [sum_{h<g} ks[h], +ks[g]).
 *  m, n         : output sizes, both multiples of 4 (the scales carry no padding).  m == 0 or
 *                 n == 0 is a no-op.
 *  a, lda       : A E4M3 [m, sum(ks)], element (i, kk) at a[i*lda + kk]; lda >= sum(ks),
 *                 lda % 16 == 0, 16-byte aligned.  b, ldb: B E4M3 [n, sum(ks)], the same rules.
 *  sfa, sfb     : FP32 [sum(ks)/128, m] and [sum(ks)/128, n], row-major (block b of row i at
 *                 sfa[b*m + i]): one scale per row and 128-long K block on both sides;
 *                 16-byte aligned.
 *  c, d         : FP32 [num_groups, m, n], contiguous (group g at + g*m*n); c must not be NULL
 *                 and may equal d (in-place accumulation; otherwise C is read, D written).
 * Every group is validated before any work is queued.  Returns DG_OK or a negative dg_status.
 */
int dg_k_grouped_fp8_gemm_nt_contiguous(int32_t num_groups, int32_t m, int32_t n, const int32_t* ks,
                                        const void* a, int64_t lda, const float* sfa,
                                        const void* b, int64_t ldb, const float* sfb,
                                        const float* c, float* d, hipStream_t stream);

/*
 * K-grouped contiguous GEMM with both operands stored K-outermost (page "第13章 DeepGEMM"
 * §13.6 and §13.13: k_grouped_fp8_gemm_tn_contiguous, the weight-gradient form whose operands
 * are the token-major activations and output gradients as the forward pass leaves them):
 *  a, lda : A E4M3 [sum(ks), m], element (i, kk) at a[kk*lda + i]; m <= lda < 2^23, lda % 16 == 0,
 *           sum(ks) * lda < 2^31, 16-byte aligned.
 *  b, ldb : B E4M3 [sum(ks), n], element (j, kk) at b[kk*ldb + j]; the same rules with n.
 * Scales, C, D, groups and errors as in dg_k_grouped_fp8_gemm_nt_contiguous; the same D.
 * Problems with more than 64 non-empty groups (either layout) take one launch per 64 groups.
 */
int dg_k_grouped_fp8_gemm_tn_contiguous(int32_t num_groups, int32_t m, int32_t n, const int32_t* ks,
                                        const void* a, int64_t lda, const float* sfa,
                                        const void* b, int64_t ldb, const float* sfb,
                                        const float* c, float* d, hipStream_t stream);

/*
 * Per-token-group FP8 cast (page "02 · DeepGEMM 技术解析" §1.1: activations in 1x128 groups
 * along K, one FP32 scale per group; page "第13章 DeepGEMM" §13.3: the scale is amax / 448):
 * produces the A operand and its scales for the GEMMs above, already in their layout.
 *
 *   s[r, b] = max_{k in group b} |x[r, k]| / 448   (FP32; 1 for an all-zero group)
 *   q[r, k] = E4M3(clamp(x[r, k] / s[r, b], -448, 448)), rounded to nearest, ties to even
 *
 * Both divisions are correctly rounded FP32 divisions.
 *  x, ldx, x_dtype : BF16 or FP32 [m, k], row stride ldx elements; rows and start 16-byte aligned.
 *  q, ldq          : E4M3 codes [m, k] (uint8), row stride ldq (a multiple of 8), 8-byte aligned.
 *  sf, sf_stride   : the scales, MN-major with sf_stride == align4(m) (what dg_fp8_gemm_nt takes
 *                    as sfa in the same sf_format).  Padding rows [m, align4(m)) are not written.
 *  sf_format       : DG_SF_F32: FP32 s[r, b] at sf[b*sf_stride + r], 4-byte aligned.
 *                    DG_SF_UE8M0X4 (scales restricted to powers of two, page
 *                    "02 · DeepGEMM 技术解析" §3.1): s[r, b] is amax / 448 (FP32) raised to the
 *                    next power of two (1 for an all-zero group, at least 2^-126), so every
 *                    quotient stays within +-448; its 8-bit exponent code goes to byte b % 4 of
 *                    int32 word (r, b / 4) at sf[(b/4)*sf_stride + r] (bytes past the last group
 *                    are 0), sf 4-byte aligned.  The codes equal dg_transform_sf's packing of
 *                    the same scales.
 *  k must be a positive multiple of 128.  m == 0 is a no-op (pointers may be NULL).
 *  Non-finite inputs give unspecified codes and scales.
 */
int dg_per_token_group_cast_fp8(int32_t m, int32_t k, const void* x, int64_t ldx, int32_t x_dtype,
                                void* q, int64_t ldq, void* sf, int64_t sf_stride, int32_t sf_format,
                                hipStream_t stream);

/*
 * Scale-layout transform (page "02 · DeepGEMM 技术解析" §3.1 and §3.2; page "第13章
 * DeepGEMM" §13.3, second constraint): converts FP32 scales to the MN-major, 16-byte
 * aligned layout the GEMMs read, optionally broadcasting 128-row blocks to every row and
 * packing UE8M0 codes four per int32.
 *
 *  sf_in        : FP32 [num_groups, ceil(mn / gran_mn), sf_k], K-major, contiguous.
 *  gran_mn      : 1 (one scale per row) or 128 (one per 128-row block, broadcast per row).
 *  pack_ue8m0   : 0 -> sf_out is FP32 [num_groups, sf_k, align4(mn)]:
 *                      element (r, b) of group g at g*sf_k*align4(mn) + b*align4(mn) + r.
 *                 1 -> sf_out is int32 [num_groups, packed_sf_k, align4(mn)]: word (r, q) holds
 *                      the UE8M0 codes of K-blocks 4q..4q+3 of row r, byte t = block 4q+t.
 *                      The code of an FP32 scale is its exponent field, (bits >> 23) & 0xff:
 *                      the mantissa is dropped (0.75 -> 0.5, 3 -> 2).
 *                 Padding rows [mn, align4(mn)) and tail bytes (4q+t >= sf_k) are written 0.
 *  mn == 0 is a no-op (pointers may be NULL).
 *  nonpow2_count: NULL, or device int32; when packing, the number of input scales that are
 *                 not exact powers of two ((bits & 0x807fffff) != 0) is ADDED to it (the
 *                 caller zeroes it).  The library counts instead of trapping.
 */
int dg_transform_sf(const float* sf_in, int32_t num_groups, int32_t mn, int32_t sf_k,
                    int32_t gran_mn, int32_t pack_ue8m0, void* sf_out,
                    int32_t* nonpow2_count, hipStream_t stream);

/* align(mn, 16 / elem_bytes): the padded MN extent of an MN-major scale tensor whose
 * K slices start on 16-byte boundaries (page "02 · DeepGEMM 技术解析" §3.1, ALIGN_MN).
 * elem_bytes must be 1, 2, 4, 8 or 16; returns -1 otherwise. */
int64_t dg_get_tma_aligned_size(int64_t mn, int32_t elem_bytes);

/* Row alignment of each group segment in the contiguous layout: the M block, 128
 * (page "02 · DeepGEMM 技术解析" §5.1). */
int32_t dg_get_mk_alignment_for_contiguous_layout(void);

/* Persistent grid size (the number of compute units the scheduler spreads tiles over).
 * n > 0 sets it, n == 0 restores the default (the device's CU count); n < 0 is an error. */
int dg_set_num_sms(int32_t n);
int32_t dg_get_num_sms(void);

/* Tile configuration the heuristic picks, without launching anything (host only).
 *  kind: 0 dense, 1 contiguous, 2 masked.  For masked, m is m_max and expected_m the hint.
 *  num_sms: grid size to plan for (> 0).  Outputs may be NULL.  *num_tiles is the
 *  number of output tiles (masked: assuming every group has expected_m valid rows). */
int dg_get_gemm_config(int32_t kind, int32_t m, int32_t n, int32_t k, int32_t num_groups,
                       int32_t expected_m, int32_t sf_format, int32_t gran_n, int32_t d_dtype,
                       int32_t num_sms, int32_t* block_m, int32_t* block_n,
                       int32_t* num_tiles, int32_t* grid);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* dg_get_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
