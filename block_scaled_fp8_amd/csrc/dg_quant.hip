// Per-token-group FP8 cast for gfx950 (MI355X): BF16 or FP32 activations [m, k] -> E4M3
// codes [m, k] and one FP32 scale per row and 128-long K group, amax / 448, written
// MN-major with the stride align4(m) that the GEMM reads (page "02 · DeepGEMM 技术解析"
// §1.1 and §3.1; page "第13章 DeepGEMM" §13.3).
//
// An item is four consecutive groups of one row: lane l holds elements 8l..8l+7 (one
// 16-byte load for BF16, two for FP32), so 16 lanes cover a group and the group's amax is
// a 4-step xor shuffle inside those 16 lanes.  A wave loads two items before casting either
// (measured on the 4096x7168 BF16 cast: two items per wave 20.5 us, four 23.5 us, eight
// 28 us; more, smaller waves keep more loads in flight across the chip).  The scale and every
// quotient are correctly rounded FP32 divisions; the E4M3 code is rounded to nearest, ties to
// even, by the hardware conversion.  Algorithmic traffic: (2 or 4) + 1 bytes per element plus
// 4 per 128 elements (FP32 scales) or 4 per 512 (packed UE8M0 codes).
#include "dg_internal.h"

namespace dg {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// E4M3 codes of two FP32 values in [-448, 448], rounded to nearest with ties to even, into
// 16-bit half HI of `word`: gfx950's v_cvt_pk_fp8_f32 writes the OCP E4M3 format (bias 7,
// subnormals, largest 448).  Its rounding is checked bit for bit against the oracle's
// nearest-value encoder, rounding ties and subnormals included, by the parity tests.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b, uint32_t word) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)word, HI);
}

constexpr int ITEMS = 2;  // (row, chunk) items per wave, both loaded before either is cast

// UE8M0 code of the smallest power of two >= t (t >= 0 a finite FP32 scale; 1 for t == 0,
// at least 2^-126): the exponent field, plus one when any mantissa bit is set.
__device__ __forceinline__ uint32_t ue8m0_ceil(float t) {
  const uint32_t b = __float_as_uint(t);
  const uint32_t e = b >> 23;
  if (t == 0.f) return 127u;
  if (e == 0u) return 1u;
  return e + ((b & 0x7FFFFFu) != 0u);
}

// UE8M0: the scales are written as packed codes, the word of a row and item holding its four
// groups (byte t = group 4*item + t; bytes past the last group are 0), at sf[item*sf_stride + row].
template <bool BF16, bool UE8M0>
__global__ void __launch_bounds__(256) cast_kernel(const void* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q,
                                                   int64_t ldq, void* __restrict__ sf, int64_t sf_stride,
                                                   uint32_t items, uint32_t chunks, int sf_k) {
  const int lane = threadIdx.x & 63;
  // Workgroups are dealt to the eight XCDs in turn; renumber them so that each XCD takes one
  // contiguous run of items.  Neighbouring rows then share an L2, whose write-back merges
  // their 4-byte scale stores (MN-major, adjacent rows adjacent in memory) into whole lines.
  const uint32_t nb = gridDim.x, per = nb >> 3, extra = nb & 7, xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const uint32_t blk = xcd < extra ? xcd * (per + 1) + idx : extra * (per + 1) + (xcd - extra) * per + idx;
  const uint32_t w0 = (blk * 4u + (threadIdx.x >> 6)) * ITEMS;  // first (row, chunk of 4 groups)
  if (w0 >= items) return;                                              // whole waves only
  float v[ITEMS][8];
  int64_t rows[ITEMS];
  int gs[ITEMS];
  bool act[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const uint32_t w = w0 + it;
    const uint32_t row = w / chunks;
    const int chunk = (int)(w - row * chunks);
    rows[it] = row;
    gs[it] = chunk * 4 + (lane >> 4);
    act[it] = w < items && gs[it] < sf_k;  // the last chunk of a row may hold fewer than 4 groups
    const int64_t col = (int64_t)gs[it] * 128 + (lane & 15) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[it][i] = 0.f;
    if (act[it]) {
      if (BF16) {
        const v4u r = *(const v4u*)((const uint16_t*)x + rows[it] * ldx + col);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[it][2 * i] = __uint_as_float(r[i] << 16);
          v[it][2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
        }
      } else {
        const float* p = (const float*)x + rows[it] * ldx + col;
        const v4u r0 = *(const v4u*)p, r1 = *(const v4u*)(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[it][i] = __uint_as_float(r0[i]);
          v[it][4 + i] = __uint_as_float(r1[i]);
        }
      }
    }
  }
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[it][i]));
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));  // within 16 lanes
    float s = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.f);
    uint32_t code = 0;
    if constexpr (UE8M0) {
      code = ue8m0_ceil(s);
      s = __uint_as_float(code << 23);
    }
    // v / s correctly rounded, from the correctly rounded reciprocal y: q0 = v*y is within an
    // ulp, the FMA gives its exact remainder, and one more FMA rounds correctly (Markstein's
    // theorem).  Three instructions instead of a full division per element; a scale so small
    // that 1/s would overflow takes the plain division.
    const float y = __fdiv_rn(1.f, s);
    const bool fast = s >= 0x1p-100f;
    auto quot = [&](float xv) -> float {
      if (fast) {
        const float q0 = xv * y;
        return __builtin_fmaf(__builtin_fmaf(-q0, s, xv), y, q0);
      }
      return __fdiv_rn(xv, s);
    };
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = fminf(fmaxf(quot(v[it][i]), -448.f), 448.f);
    uint32_t lo = e4m3_pair<false>(c[0], c[1], 0u), hi = e4m3_pair<false>(c[4], c[5], 0u);
    lo = e4m3_pair<true>(c[2], c[3], lo);
    hi = e4m3_pair<true>(c[6], c[7], hi);
    if (act[it]) {
      const int64_t col = (int64_t)gs[it] * 128 + (lane & 15) * 8;
      *(v2u*)(q + rows[it] * ldq + col) = (v2u){lo, hi};
      if (!UE8M0 && (lane & 15) == 0) ((float*)sf)[(int64_t)gs[it] * sf_stride + rows[it]] = s;
    }
    if constexpr (UE8M0) {
      // the four groups' codes into lane 0's word (inactive groups contribute 0)
      const uint32_t mine = act[it] ? code : 0u;
      const uint32_t word = __shfl(mine, 0) | (__shfl(mine, 16) << 8) | (__shfl(mine, 32) << 16) |
                            (__shfl(mine, 48) << 24);
      const uint32_t w = w0 + it;
      if (lane == 0 && w < items) {
        const uint32_t chunk = w - (uint32_t)rows[it] * chunks;
        ((uint32_t*)sf)[(int64_t)chunk * sf_stride + rows[it]] = word;
      }
    }
  }
}

}  // namespace

hipError_t launch_cast(const void* x, int64_t ldx, bool bf16, uint8_t* q, int64_t ldq, void* sf, int64_t sf_stride,
                       bool ue8m0, int m, int k, hipStream_t stream) {
  const int sf_k = k / 128;
  const int chunks = (sf_k + 3) / 4;
  const int64_t items = (int64_t)m * chunks;
  const int64_t waves = (items + ITEMS - 1) / ITEMS;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks * 4 * ITEMS > 0xFFFFFFFFll) return hipErrorInvalidValue;  // item indices are 32-bit
#define DG_CAST(B, U)                                                                                     \
  if (bf16 == B && ue8m0 == U)                                                                          \
    hipLaunchKernelGGL((cast_kernel<B, U>), dim3((unsigned)blocks), dim3(256), 0, stream, x, ldx, q, ldq, sf, \
                       sf_stride, (uint32_t)items, (uint32_t)chunks, sf_k);
  DG_CAST(true, false)
  DG_CAST(false, false)
  DG_CAST(true, true)
  DG_CAST(false, true)
#undef DG_CAST
  return hipGetLastError();
}

}  // namespace dg
