// Scale-layout transform kernel (page "02 · DeepGEMM 技术解析" §3.1-3.2; page
// "第13章 DeepGEMM" §13.3, second constraint).
//
// One thread per output word: word c (a K block, or a packed group of four) of row r of
// group g sits at ((g * cols + c) * align4(mn) + r), the thread's own index, so every store
// instruction of a wave writes 64 consecutive words and the grid covers every CU even for a
// single group.  Packing keeps the FP32 exponent field, (bits >> 23) & 0xff, four codes per
// int32 with byte t = K block 4q + t.
#include "dg_internal.h"

namespace dg {

__global__ void __launch_bounds__(256) transform_sf_kernel(const float* __restrict__ in, int num_groups,
                                                           int mn, int sf_k, int gran, int pack,
                                                           void* __restrict__ out, int32_t* count) {
  const int a4 = (mn + 3) & ~3;
  const int cols = pack ? (sf_k + 3) / 4 : sf_k;  // output rows of one group
  const int64_t per_g = (int64_t)cols * a4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool inside = idx < (int64_t)num_groups * per_g;
  const int g = inside ? (int)(idx / per_g) : 0;
  const int64_t rem = idx - (int64_t)g * per_g;
  const int c = inside ? (int)(rem / a4) : 0;
  const int r = inside ? (int)(rem - (int64_t)c * a4) : 0;
  const int mnb = (mn + gran - 1) / gran;
  const bool live = inside && r < mn;
  const float* src = in + ((int64_t)g * mnb + (live ? r / gran : 0)) * sf_k;
  if (!pack) {
    if (inside) ((float*)out)[idx] = live ? src[c] : 0.f;
    return;
  }
  const bool counts = live && (r % gran) == 0;  // each input scale is counted once
  int bad = 0;
  unsigned int w = 0;
  if (live) {
    for (int t = 0; t < 4; ++t) {
      const int kb = 4 * c + t;
      if (kb < sf_k) {
        const unsigned int bits = __float_as_uint(src[kb]);
        w |= ((bits >> 23) & 0xFFu) << (8 * t);
        if (counts && (bits & 0x807FFFFFu) != 0u) ++bad;
      }
    }
  }
  if (inside) ((unsigned int*)out)[idx] = w;
  if (count != nullptr) {
    // one atomic per wave (every lane of the wave takes part in the sum, inside or not)
    for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d);
    if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(count, bad);
  }
}

hipError_t launch_transform_sf(const float* in, int num_groups, int mn, int sf_k, int gran_mn, int pack,
                               void* out, int32_t* count, hipStream_t stream) {
  const int64_t words = (int64_t)num_groups * (pack ? (sf_k + 3) / 4 : sf_k) * ((mn + 3) & ~3);
  if (words == 0) return hipSuccess;
  const int64_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(transform_sf_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, num_groups, mn,
                     sf_k, gran_mn, pack, out, count);
  return hipGetLastError();
}

}  // namespace dg
