// Skinny (decode-shaped) block-scaled FP8 GEMM for gfx950: dense problems with at most 64
// rows and 128x128 FP32 weight scales ("1d2d").
//
// Computes D = C + A . B^T exactly as the other kernels do (one activation scale per row and
// 128-long K block, one weight scale per 128x128 block; each block's partial product promoted
// into an FP32 accumulator as final += scale_a * scale_b * partial: page "02 · DeepGEMM
// 技术解析" §2.2, page "第13章 DeepGEMM" §13.3 algorithm box).  With so few rows the work is
// bound by streaming B from HBM once (page "02 · DeepGEMM 技术解析" §5.2 frames decode as the
// latency-critical case), so the kernel is organised for memory-level parallelism instead of
// operand reuse:
//  * a workgroup owns every row (<= 64) and BN (16 or 32) columns; its NW waves split K, wave w
//    taking K blocks w, w + NW, ...;
//  * operand fragments go from global memory straight into registers (no LDS staging); a wave
//    issues the loads of two K blocks before it computes either, so every wave has two blocks
//    of loads outstanding from the start;
//  * at the end the waves' partial sums (each exact up to FP32 rounding of its own blocks) are
//    added through LDS, C is added, and the tile is stored row-contiguously.
// The column block of a workgroup lies inside one 128-wide weight-scale block (BN divides 128),
// so the weight scale of a K block is one scalar.
#include "dg_internal.h"

namespace dg {
namespace skinny {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int BK = 128;
constexpr int FM = 4;  // 16-row fragments: up to 64 rows

// Buffer descriptor over [base, base + bytes): reads at offsets >= bytes return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ unsigned int pack_bf16x2(float x, float y) {
  v2bf v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(unsigned int, v);
}

template <int FN>
struct Blk {
  v4u a[FM][2];  // activation fragments: rows 16i + lr, K bytes 32 lg .. 32 lg + 31 of the block
  v4u b[FN][2];  // weight fragments: rows n0 + 16j + lr, the same K bytes
  float sa[FM];  // activation scales of rows 16i + lr
  float sb;      // the weight-block scale
};

template <int BN, int NW, int OUT>
__global__ void __launch_bounds__(NW * 64) skinny_kernel(const GemmParams p) {
  constexpr int FN = BN / 16;
  constexpr int RS = BN + 4;  // LDS row stride of the partial sums, in floats
  __shared__ __attribute__((aligned(16))) float red[NW * 64 * RS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * BN;
  const int nkb = p.sf_k;
  const int m = p.m;

  // A rows 0..m-1 and B rows n0..n0+BN-1 that exist; anything past them reads as zero
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.a, (uint32_t)m * (uint32_t)p.lda);
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.b + (int64_t)n0 * p.ldb, (uint32_t)min(BN, p.n - n0) * (uint32_t)p.ldb);
  const __amdgpu_buffer_rsrc_t rs = rsrc(p.sfa, (uint32_t)(4 * p.sfa_stride * nkb));
  const float* sbp = (const float*)p.sfb + (int64_t)(n0 / 128) * p.sfb_stride;
  const uint32_t offa = (uint32_t)lr * (uint32_t)p.lda + 32u * (uint32_t)lg;
  const uint32_t offb = (uint32_t)lr * (uint32_t)p.ldb + 32u * (uint32_t)lg;
  const uint32_t stepa = 16u * (uint32_t)p.lda, stepb = 16u * (uint32_t)p.ldb;

  auto load = [&](Blk<FN>& s, int kb) {
    const uint32_t kofs = (uint32_t)kb * BK;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) s.a[i][h] = __builtin_amdgcn_raw_buffer_load_b128(ra, offa + i * stepa + kofs + 16 * h, 0, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) s.b[j][h] = __builtin_amdgcn_raw_buffer_load_b128(rb, offb + j * stepb + kofs + 16 * h, 0, 0);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // rows past m read row 0's (finite) scale: their operands are zero and they are never
      // stored, and leaving the loaded value untouched here keeps the loads in flight
      const int row = 16 * i + lr;
      s.sa[i] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * (uint32_t)(kb * (int)p.sfa_stride + (row < m ? row : 0)), 0, 0));
    }
    s.sb = ((const __attribute__((address_space(4))) float*)sbp)[kb];
  };

  float fin[FM][FN][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) fin[i][j][v] = 0.f;

  auto compute = [&](const Blk<FN>& s) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const v8i af = {(int)s.a[i][0].x, (int)s.a[i][0].y, (int)s.a[i][0].z, (int)s.a[i][0].w,
                      (int)s.a[i][1].x, (int)s.a[i][1].y, (int)s.a[i][1].z, (int)s.a[i][1].w};
      const float f = s.sa[i] * s.sb;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v8i bf = {(int)s.b[j][0].x, (int)s.b[j][0].y, (int)s.b[j][0].z, (int)s.b[j][0].w,
                        (int)s.b[j][1].x, (int)s.b[j][1].y, (int)s.b[j][1].z, (int)s.b[j][1].w};
        // weight fragment first: a lane owns one output row (16i + lr) and four consecutive
        // columns (16j + 4lg ..)
        const v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[i][j][v] = __builtin_fmaf(f, acc[v], fin[i][j][v]);
      }
    }
  };

  // Rounds of two K blocks per wave (blocks r + wave and r + NW + wave): both blocks' loads go
  // out unconditionally (a block past the end re-reads the last one and is not computed), so
  // the first block's MFMAs wait only for their own loads while the second's are in flight.
  for (int r = 0; r < nkb; r += 2 * NW) {
    const int k0 = r + wave, k1 = r + NW + wave;
    Blk<FN> s0, s1;
    load(s0, min(k0, nkb - 1));
    __builtin_amdgcn_sched_barrier(0);  // (all of block k0's loads go out before block k1's)
    load(s1, min(k1, nkb - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (k0 < nkb) compute(s0);
    if (k1 < nkb) compute(s1);
  }

  // partial sums of every wave -> LDS; each wave writes its 64 x BN partial tile
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      *(v4f*)(red + (wave * 64 + 16 * i + lr) * RS + 16 * j + 4 * lg) =
          (v4f){fin[i][j][0], fin[i][j][1], fin[i][j][2], fin[i][j][3]};
  __syncthreads();

  // one 4-column group per thread: sum over the waves, add C, store
  constexpr int CG = BN / 4;
  for (int t = threadIdx.x; t < 64 * CG; t += NW * 64) {
    const int row = t / CG, cg = t - row * CG;
    if (row >= m) continue;
    v4f o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) o += *(const v4f*)(red + (w * 64 + row) * RS + 4 * cg);
    const int col = n0 + 4 * cg;
    if (col >= p.n) continue;
    const bool full4 = col + 3 < p.n;
    if (OUT == OUT_F32_C) {
      const float* crow = p.c + (int64_t)row * p.ldc;
      if (full4 && p.c_vec) {
        o += *(const v4f*)(crow + col);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (col + v < p.n) o[v] += crow[col + v];
      }
    }
    if (OUT == OUT_BF16) {
      unsigned short* dp = (unsigned short*)p.d + (int64_t)row * p.ldd + col;
      const unsigned int w0 = pack_bf16x2(o[0], o[1]), w1 = pack_bf16x2(o[2], o[3]);
      if (full4 && p.d_vec) {
        *(v2u*)dp = (v2u){w0, w1};
      } else {
        const unsigned short h[4] = {(unsigned short)w0, (unsigned short)(w0 >> 16), (unsigned short)w1,
                                     (unsigned short)(w1 >> 16)};
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (col + v < p.n) dp[v] = h[v];
      }
    } else {
      float* dp = (float*)p.d + (int64_t)row * p.ldd + col;
      if (full4 && p.d_vec) {
        *(v4f*)dp = o;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (col + v < p.n) dp[v] = o[v];
      }
    }
  }
}

template <int BN, int NW, int OUT>
static hipError_t launch_nw(const GemmParams& p, hipStream_t s) {
  const int grid = (p.n + BN - 1) / BN;
  hipLaunchKernelGGL((skinny_kernel<BN, NW, OUT>), dim3(grid), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

// (8 waves per workgroup measured best: 4 leave less memory-level parallelism, 16 run out of
// registers)
template <int BN, int OUT>
static hipError_t launch_one(const GemmParams& p, hipStream_t s) {
  return launch_nw<BN, 8, OUT>(p, s);
}

}  // namespace skinny

// Dense problems with m <= 64 rows and 1d2d FP32 scales; bn: 16 or 32 columns per workgroup.
hipError_t launch_skinny(const GemmParams& p, int bn, int out, hipStream_t stream) {
  if (p.m > 64 || p.m <= 0) return hipErrorInvalidValue;
#define DG_CASE(BN, O) \
  if (bn == BN && out == O) return skinny::launch_one<BN, O>(p, stream);
  DG_CASE(16, OUT_BF16)
  DG_CASE(16, OUT_F32)
  DG_CASE(16, OUT_F32_C)
  DG_CASE(32, OUT_BF16)
  DG_CASE(32, OUT_F32)
  DG_CASE(32, OUT_F32_C)
#undef DG_CASE
  return hipErrorInvalidValue;
}

}  // namespace dg
