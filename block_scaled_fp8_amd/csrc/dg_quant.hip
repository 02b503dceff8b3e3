// Per-token-group FP8 cast for gfx950 (MI355X): BF16 or FP32 activations [m, k] -> E4M3
// codes [m, k] and one FP32 scale per row and 128-long K group, amax / 448, written
// MN-major with the stride align4(m) that the GEMM reads (page "02 · DeepGEMM 技术解析"
// §1.1 and §3.1; page "第13章 DeepGEMM" §13.3).
//
// One wave casts four consecutive groups of one row: lane l holds elements 8l..8l+7 (one
// 16-byte load for BF16, two for FP32), so 16 lanes cover a group and the group's amax is
// a 4-step xor shuffle inside those 16 lanes.  The scale and every quotient are correctly
// rounded FP32 divisions; the E4M3 code is rounded to nearest, ties to even, from the FP32
// bits.  HBM-bound: (2 or 4) + 1 bytes per element plus 4 per 128 elements.
#include "dg_internal.h"

namespace dg {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// OCP E4M3 (bias 7, subnormals, largest 448) code of a finite FP32 value with |v| <= 448,
// rounded to nearest with ties to even.  The sign goes to bit 7.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a < 0.015625f) {  // below 2^-6: a multiple of 2^-9; a * 512 is exact, rint ties to even
    return sign | (uint32_t)rintf(a * 512.0f);  // 8 lands on the smallest normal, code 0x08
  }
  const uint32_t ab = __float_as_uint(a);
  uint32_t e = (ab >> 23) - 127u + 7u;  // 1..15
  uint32_t m = (ab >> 20) & 7u;
  const uint32_t rest = ab & 0xFFFFFu;  // the 20 mantissa bits below the kept three
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
  if (m == 8u) {
    m = 0u;
    ++e;
  }
  return sign | (e << 3) | m;  // |v| <= 448 keeps this at or below 0x7E
}

template <bool BF16>
__global__ void __launch_bounds__(256) cast_kernel(const void* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q,
                                                   int64_t ldq, float* __restrict__ sf, int64_t sf_stride,
                                                   int64_t waves, int chunks, int sf_k) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, chunk of 4 groups)
  if (w >= waves) return;                                          // whole waves only
  const int64_t row = w / chunks;
  const int chunk = (int)(w - row * chunks);
  const int g = chunk * 4 + (lane >> 4);
  const bool active = g < sf_k;  // the last chunk of a row may hold fewer than 4 groups
  const int64_t col = (int64_t)g * 128 + (lane & 15) * 8;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  if (active) {
    if (BF16) {
      const v4u r = *(const v4u*)((const uint16_t*)x + row * ldx + col);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(r[i] << 16);
        v[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
      }
    } else {
      const float* p = (const float*)x + row * ldx + col;
      const v4u r0 = *(const v4u*)p, r1 = *(const v4u*)(p + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = __uint_as_float(r0[i]);
        v[4 + i] = __uint_as_float(r1[i]);
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));  // within 16 lanes
  const float s = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.f);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3_rne(fminf(fmaxf(__fdiv_rn(v[i], s), -448.f), 448.f)) << (8 * i);
    hi |= e4m3_rne(fminf(fmaxf(__fdiv_rn(v[4 + i], s), -448.f), 448.f)) << (8 * i);
  }
  if (active) {
    *(v2u*)(q + row * ldq + col) = (v2u){lo, hi};
    if ((lane & 15) == 0) sf[(int64_t)g * sf_stride + row] = s;
  }
}

}  // namespace

hipError_t launch_cast(const void* x, int64_t ldx, bool bf16, uint8_t* q, int64_t ldq, float* sf, int64_t sf_stride,
                       int m, int k, hipStream_t stream) {
  const int sf_k = k / 128;
  const int chunks = (sf_k + 3) / 4;
  const int64_t waves = (int64_t)m * chunks;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(cast_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x, ldx, q, ldq, sf,
                       sf_stride, waves, chunks, sf_k);
  else
    hipLaunchKernelGGL(cast_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x, ldx, q, ldq, sf,
                       sf_stride, waves, chunks, sf_k);
  return hipGetLastError();
}

}  // namespace dg
