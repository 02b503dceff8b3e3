// Internal interface between the host library (dg_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// How the weight scales are laid out and applied (page "02 · DeepGEMM 技术解析" §2.3).
enum SfMode {
  SF_1D2D_F32 = 0,    // sfa FP32 MN-major per row; sfb FP32 per 128x128 block, K-major
  SF_1D1D_F32 = 1,    // sfa and sfb FP32 MN-major, one scale per row and K block
  SF_1D1D_UE8M0 = 2,  // sfa and sfb UE8M0 packed four per int32, MN-major
  // FP4 (E2M1) weights, two per byte (page "第13章 DeepGEMM" §13.5): sfa UE8M0 per row and 128-K
  // block packed four per int32 as above; sfb UE8M0 per row and 32-K block, the four codes of
  // one 128-K block in one int32 (byte t = 32-block t), MN-major [k / 128][align4(n)]
  SF_FP4_UE8M0 = 3,
};

// GRP_KGROUP: the K-grouped form (groups concatenated along K, one output per group)
enum GroupMode { GRP_DENSE = 0, GRP_CONTIG = 1, GRP_MASKED = 2, GRP_KGROUP = 3 };

// K-grouped problems with at most this many non-empty groups run in one launch
constexpr int kMaxKGroups = 64;

enum OutMode { OUT_BF16 = 0, OUT_F32 = 1, OUT_F32_C = 2 };

// Operand storage (page "第13章 DeepGEMM" §13.3: the two letters of fp8_gemm_{nt,nn,tn,tt}):
// LAYOUT_A_MN: A stored [K, M] (element (i, kk) at a[kk*lda + i]); LAYOUT_B_MN: B stored [K, N]
// (element (j, kk) at b[kk*ldb + j]).  0 is the NT form, both operands K-major.
enum LayoutBits { LAYOUT_A_MN = 1, LAYOUT_B_MN = 2 };

// Everything a GEMM launch needs.  Sizes in elements; pointers are device memory.
struct GemmParams {
  const uint8_t* a;
  int64_t lda, a_gstride;
  const void* sfa;
  int64_t sfa_stride, sfa_gstride;
  const uint8_t* b;
  int64_t ldb, b_gstride;
  const void* sfb;
  int64_t sfb_stride, sfb_gstride;
  const float* c;
  int64_t ldc;
  void* d;
  int64_t ldd, d_gstride;
  const int32_t* grouped_layout;  // contiguous mode
  const int32_t* masked_m;        // masked mode
  int32_t m;                      // dense: M; contiguous: total rows; masked: m_max
  int32_t n, k, num_groups;
  int32_t sf_k;
  int32_t num_m_tiles;            // dense / contiguous (masked: per group, from m_max)
  int32_t num_n_tiles;
  int32_t total_tiles;            // dense / contiguous; masked computes it on the device
  int32_t swizzle_m;              // m tiles per swizzle super-row
  int32_t xcd_remap;              // 1: map consecutive logical workgroups onto one XCD
  int32_t d_vec;                  // 1: D rows allow 4-element vector stores (ldd % 4 == 0, 16-B base)
  int32_t c_vec;                  // 1: C rows allow 4-element vector loads
  int32_t d_vec16;                // 1: D rows and base are 16-byte aligned
  int32_t layout;                 // LayoutBits (pipelined kernel only)
  // K-grouped: C between groups, and the non-empty groups in order (output index, first
  // 128-long K block, number of K blocks); num_m_tiles * num_n_tiles tiles per group
  int64_t c_gstride;
  int32_t kg_count;
  int32_t kg_group[kMaxKGroups];
  int32_t kg_kb0[kMaxKGroups];
  int32_t kg_nkb[kMaxKGroups];
};

struct TileCfg {
  int bm, bn, wm, wn;  // workgroup tile, waves along M and N
};

constexpr int kNumTiles = 9;
extern const TileCfg kTiles[kNumTiles];

// Launch the GEMM kernel instantiated for (tile, sf_mode, group, out).  Returns
// hipErrorInvalidValue for a combination that is not instantiated.
hipError_t launch_gemm(const GemmParams& p, int tile, int sf_mode, int group, int out, int grid,
                       hipStream_t stream);
bool gemm_instantiated(int tile, int sf_mode, int group, int out, int layout = 0);
int gemm_lds_bytes(int tile);

// Deep-pipelined kernels (dg_gemm_pipe.hip): dense problems, contiguous and masked groups.
// A tile needs at least pipe_stages_b(bm, bn, group) K blocks.
bool pipe_instantiated(int bm, int bn, int sf_mode, int group, int out, int layout = 0);
int pipe_stages_b(int bm, int bn, int group);
int pipe_lds_bytes(int bm, int bn, int sf_mode, int group);
hipError_t launch_pipe(const GemmParams& p, int bm, int bn, int sf_mode, int group, int out, int grid,
                       hipStream_t stream);
// (dg_gemm_pipe.hip is compiled in parts, one per group of instantiations)
hipError_t launch_pipe_dense(const GemmParams& p, int bm, int bn, int sf_mode, int out, int grid, hipStream_t s);
hipError_t launch_pipe_contig(const GemmParams& p, int bm, int bn, int sf_mode, int out, int grid, hipStream_t s);
hipError_t launch_pipe_masked(const GemmParams& p, int bm, int bn, int sf_mode, int out, int grid, hipStream_t s);
hipError_t launch_pipe_fp4(const GemmParams& p, int bm, int bn, int group, int out, int grid, hipStream_t s);
// operands stored MN-major (p.layout != 0): one part per layout (A, B, both)
hipError_t launch_pipe_layout(const GemmParams& p, int bm, int bn, int sf_mode, int group, int out, int grid,
                              hipStream_t s);
hipError_t launch_pipe_layout_b(const GemmParams& p, int bm, int bn, int sf_mode, int group, int out, int grid,
                                hipStream_t s);
hipError_t launch_pipe_layout_ab(const GemmParams& p, int bm, int bn, int sf_mode, int group, int out, int grid,
                                 hipStream_t s);

// Skinny kernel (dg_gemm_skinny.hip): dense problems with 1 <= m <= 64 rows and 1d2d FP32
// scales, bn (16 or 32) columns per workgroup, the workgroup's waves splitting K.
hipError_t launch_skinny(const GemmParams& p, int bn, int out, hipStream_t stream);

hipError_t launch_cast(const void* x, int64_t ldx, bool bf16, uint8_t* q, int64_t ldq, void* sf, int64_t sf_stride,
                       bool ue8m0, int m, int k, hipStream_t stream);

hipError_t launch_transform_sf(const float* in, int num_groups, int mn, int sf_k, int gran_mn,
                               int pack, void* out, int32_t* count, hipStream_t stream);

}  // namespace dg
