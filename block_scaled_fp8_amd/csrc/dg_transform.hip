// Scale-layout transform kernel (page "02 · DeepGEMM 技术解析" §3.1-3.2; page
// "第13章 DeepGEMM" §13.3, second constraint).
//
// One thread per output row r of the MN-major layout (including the padding rows
// up to align4(mn)); it walks the K blocks, so every store instruction of a wave
// writes 64 consecutive words.  Packing keeps the FP32 exponent field,
// (bits >> 23) & 0xff, four codes per int32 with byte t = K block 4q + t.
#include "dg_internal.h"

namespace dg {

__global__ void __launch_bounds__(256) transform_sf_kernel(const float* __restrict__ in, int num_groups,
                                                           int mn, int sf_k, int gran, int pack,
                                                           void* __restrict__ out, int32_t* count) {
  const int a4 = (mn + 3) & ~3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_groups * a4) return;
  const int g = (int)(idx / a4);
  const int r = (int)(idx - (int64_t)g * a4);
  const int mnb = (mn + gran - 1) / gran;
  const bool live = r < mn;
  const float* src = in + ((int64_t)g * mnb + (live ? r / gran : 0)) * sf_k;
  if (!pack) {
    float* o = (float*)out + (int64_t)g * sf_k * a4 + r;
    for (int kb = 0; kb < sf_k; ++kb) {
      float v = 0.f;
      if (live) v = src[kb];
      o[(int64_t)kb * a4] = v;
    }
    return;
  }
  const int pk = (sf_k + 3) / 4;
  unsigned int* o = (unsigned int*)out + (int64_t)g * pk * a4 + r;
  const bool counts = live && (r % gran) == 0;  // each input scale is counted once
  int bad = 0;
  for (int q = 0; q < pk; ++q) {
    unsigned int w = 0;
    if (live) {
      for (int t = 0; t < 4; ++t) {
        const int kb = 4 * q + t;
        if (kb < sf_k) {
          const unsigned int bits = __float_as_uint(src[kb]);
          w |= ((bits >> 23) & 0xFFu) << (8 * t);
          if (counts && (bits & 0x807FFFFFu) != 0u) ++bad;
        }
      }
    }
    o[(int64_t)q * a4] = w;
  }
  if (count != nullptr && bad != 0) atomicAdd(count, bad);
}

hipError_t launch_transform_sf(const float* in, int num_groups, int mn, int sf_k, int gran_mn, int pack,
                               void* out, int32_t* count, hipStream_t stream) {
  const int64_t rows = (int64_t)num_groups * ((mn + 3) & ~3);
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + 255) / 256;
  hipLaunchKernelGGL(transform_sf_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, num_groups, mn,
                     sf_k, gran_mn, pack, out, count);
  return hipGetLastError();
}

}  // namespace dg
