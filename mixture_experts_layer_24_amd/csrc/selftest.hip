// Device self-test of the hardware E4M3 conversion the quantizers use.
//
// Every finite fp32 x with |x| <= 464 (a quantizer passes |v / s| <= 448
// (1 + 2^-23)) is encoded by e4m3x2 / e4m3x4 and by the bit-manipulation
// encoder f32_to_e4m3; the pairs and quadruples use x, -3x/4, x/4 and -x
// (all within the same range), so the byte order of the packed forms is
// checked too.  A second kernel checks the quotient encoder (e4m3x4_quot)
// against the division on 2^30 hashed quadruples.  The number of
// disagreements of both is added to *mismatches.
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

// The quotient encoder e4m3x4_quot against the division it replaces, on
// hashed quadruples as the quantizers form them: four bf16 values (every
// finite bf16 pattern, subnormals included), amax at least their largest
// magnitude (their own maximum, or that times a hashed factor, or a power
// of two times 448 so that s is a power of two and quotients land exactly on
// E4M3 rounding boundaries), s = amax / 448 (1 when amax = 0).
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du;
  x ^= x >> 15; x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__device__ __forceinline__ float finite_bf16(uint32_t h) {
  uint32_t b = h & 0xFFFFu;
  if (((b >> 7) & 0xFFu) == 0xFFu) b &= 0x807Fu;  // infinity / NaN -> a subnormal
  return __uint_as_float(b << 16);
}
__global__ void __launch_bounds__(256) quot_selftest_kernel(uint32_t base,
                                                             unsigned long long* __restrict__ mismatches) {
  const uint32_t i = base + blockIdx.x * 256u + threadIdx.x;
  const uint32_t h0 = mix32(i * 4u + 0x9e3779b9u), h1 = mix32(h0 + 1u), h2 = mix32(h1 + 2u);
  const uint32_t h3 = mix32(h2 + 3u), h4 = mix32(h3 + 4u);
  float v[4] = {finite_bf16(h0), finite_bf16(h0 >> 16), finite_bf16(h1), finite_bf16(h1 >> 16)};
  if (h4 & 1u) {  // a narrower exponent spread: values of one row are rarely 2^100 apart
    const uint32_t ex = 100u + (h4 >> 1) % 56u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = __uint_as_float((__float_as_uint(v[j]) & 0x807FFFFFu) | (((ex + j * ((h2 >> (8 * j)) & 7u)) & 0xFFu) << 23));
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[j]));
  switch (h3 & 3u) {
    case 0: break;
    case 1: amax *= 1.0f + float(h3 >> 8) * 0x1p-22f; break;   // up to x5
    case 2: {                                                   // 448 * 2^e >= amax
      int e;
      frexpf(amax / 448.0f, &e);
      amax = amax > 0.f ? ldexpf(448.0f, e) : 0.f;
      break;
    }
    default: amax = fminf(amax * 2.0f, 3.0e38f); break;
  }
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  const QuotScale q = quot_scale(s);
  const uint32_t got = e4m3x4_quot(v[0], v[1], v[2], v[3], q);
  const uint32_t want = e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
  if (got != want) atomicAdd(mismatches, 1ull);
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
  // 2^30 hashed quadruples for the quotient encoder
  for (uint32_t l = 0; l < 64; ++l)
    hipLaunchKernelGGL(quot_selftest_kernel, dim3(1u << 16), dim3(256), 0, s, l << 24, mismatches);
  return launch_status();
}

}  // namespace moe_launch
