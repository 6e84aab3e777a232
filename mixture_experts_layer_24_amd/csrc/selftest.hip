// Device self-test of the hardware E4M3 conversion the quantizers use.
//
// Every finite fp32 x with |x| <= 464 (a quantizer passes |v / s| <= 448
// (1 + 2^-23)) is encoded by e4m3x2 / e4m3x4 and by the bit-manipulation
// encoder f32_to_e4m3; the pairs and quadruples use x, -3x/4, x/4 and -x
// (all within the same range), so the byte order of the packed forms is
// checked too.  The number of disagreements is added to *mismatches.
#include "common.h"

namespace moe {

__global__ void __launch_bounds__(256) fp8_selftest_kernel(uint32_t base,
                                                            unsigned long long* __restrict__ mismatches) {
  const uint32_t i = base + blockIdx.x * 256u + threadIdx.x;
  const float x = __uint_as_float(i);
  if (!(fabsf(x) <= 464.f)) return;  // NaN, infinities and the unused range
  const float y = -0.75f * x, z = 0.25f * x, w = -x;
  const uint32_t want2 = f32_to_e4m3(x) | (f32_to_e4m3(y) << 8);
  const uint32_t want4 = want2 | (f32_to_e4m3(z) << 16) | (f32_to_e4m3(w) << 24);
  const unsigned long long bad = (e4m3x2(x, y) != want2) + (e4m3x4(x, y, z, w) != want4);
  if (bad) atomicAdd(mismatches, bad);
}

__global__ void zero_u64_kernel(unsigned long long* p) { *p = 0ull; }

}  // namespace moe

namespace moe_launch {
using namespace moe;

int fp8_convert_selftest(unsigned long long* mismatches, hipStream_t s) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, s, mismatches);
  // 2^32 patterns in 256 launches of 2^24 (a grid dimension holds < 2^32 threads)
  for (uint32_t l = 0; l < 256; ++l)
    hipLaunchKernelGGL(fp8_selftest_kernel, dim3(1u << 16), dim3(256), 0, s, l << 24, mismatches);
  return launch_status();
}

}  // namespace moe_launch
