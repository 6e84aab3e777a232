// Internal definitions shared by the HIP kernels of the MoE expert layer.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA matrix cores, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---- OCP E4M3FN encode: round to nearest even, saturate to +-448 ----------
// Works on the exact fp32 value: the result is the E4M3 grid point nearest
// to |v| (ties to the even code), clamped to 448.  Bit manipulation only, so
// the decision is the same on every device and in every build.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;          // |v| >= 448
  uint32_t code;
  if (a < 0x3C800000u) {                                // |v| < 2^-6: subnormal grid, step 2^-9
    // |v| / 2^-9 rounded to nearest even integer, in [0, 8]
    float q = __uint_as_float(a) * 512.0f;              // exact scaling by a power of two
    float r = __builtin_rintf(q);                       // default mode: nearest even
    code = uint32_t(r);                                 // 8 becomes the smallest normal (0x08)
  } else {
    uint32_t exp = (a >> 23) - 127 + 7;                 // biased E4M3 exponent, 1..15
    uint32_t mant = a & 0x7FFFFFu;
    uint32_t keep = mant >> 20;                         // 3 mantissa bits
    uint32_t rest = mant & 0xFFFFFu;
    uint32_t half = 0x80000u;
    uint32_t up = (rest > half) || (rest == half && (keep & 1u));
    code = ((exp << 3) | keep) + up;                    // carry rolls into the exponent
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// The same encoding by the hardware's packed conversion, two or four values
// at a time (bytes from low to high in argument order).  It rounds to
// nearest even like f32_to_e4m3 and gives the same code for every finite
// fp32 of magnitude <= 464 (moe_fp8_convert_selftest checks all of them on
// the device); the quantizers pass v / s with |v| <= amax = 448 s, so
// |v / s| <= 448 (1 + 2^-23).  One instruction per pair instead of the
// bit manipulation above, which stays the reference.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// E4M3 codes of the fp32 quotients v / s (the division rounded to nearest)
// for one scale s and four values, mostly without dividing.  With r = RN(1/s)
// the product q0 = RN(v r) is within (2^-23 + 2^-48) |v/s| of v/s, and RN(v/s)
// within 2^-24 |v/s|, so RN(v/s) lies between q0 (1 - 2^-20) and q0 (1 + 2^-20)
// (each end rounded toward q0 by at most 2^-24 relative, far inside the
// margin).  The encoding is monotone, so when both ends give the same four
// codes those are the codes of RN(v/s); otherwise (a value within ~2^-20 of
// a rounding boundary) the division decides.  Below 2^-126 the relative
// bound does not hold, but there every quotient in the interval encodes to
// a signed zero.  `fast` is false when 1/s is not a normal number, and then
// every quotient is divided.
struct QuotScale {
  float s, r;
  bool fast;
};
__device__ __forceinline__ QuotScale quot_scale(float s) {
  QuotScale q;
  q.s = s;
  q.r = 1.0f / s;
  q.fast = s >= 0x1p-125f && s <= 0x1p125f;
  return q;
}
__device__ __forceinline__ uint32_t e4m3x4_quot(float a, float b, float c, float d,
                                                const QuotScale& q) {
  if (q.fast) {
    const float qa = a * q.r, qb = b * q.r, qc = c * q.r, qd = d * q.r;
    constexpr float kLo = 1.0f - 0x1p-20f, kHi = 1.0f + 0x1p-20f;
    const uint32_t lo = e4m3x4(qa * kLo, qb * kLo, qc * kLo, qd * kLo);
    const uint32_t hi = e4m3x4(qa * kHi, qb * kHi, qc * kHi, qd * kHi);
    if (lo == hi) return lo;
  }
  return e4m3x4(a / q.s, b / q.s, c / q.s, d / q.s);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0 ? float(m) * (1.0f / 512.0f)
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | s);
}

// ---- wave reductions -----------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Per-row E4M3 quantization of a bf16 row (length a multiple of 8) by one
// wave: scale s = amax / 448 (1 for an all-zero row), codes = E4M3(v / s)
// with the division in fp32.
__device__ __forceinline__ void rowq_wave(const uint16_t* __restrict__ src, int len,
                                          uint8_t* __restrict__ dst, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  float amax = 0.f;
  for (int c = lane * 8; c < len; c += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
  }
  amax = wave_max(amax);
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (lane == 0) *scale = s;
  const QuotScale qs = quot_scale(s);
  for (int c = lane * 8; c < len; c += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + c);
    const uint32_t lo = e4m3x4_quot(bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1]), qs);
    const uint32_t hi = e4m3x4_quot(bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3]), qs);
    *reinterpret_cast<uint2*>(dst + c) = make_uint2(lo, hi);
  }
}



// Allow a kernel to use more than the default 64 KB of dynamic LDS (gfx950
// has 160 KB per CU).  Called once per kernel before its first launch.
template <typename Kernel>
inline bool allow_lds(Kernel k, size_t bytes) {
  if (bytes <= 65536) return true;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes)) == hipSuccess;
}

}  // namespace moe

// Host-side launch helpers implemented in the kernel files.
namespace moe_launch {
int route(const void* x, const void* w_gate, const float* bias, float* logits, int T, int h,
          int E, int k, int dtype, int32_t* topk_idx, float* topk_w, hipStream_t s);
int index_build(const int32_t* topk_idx, int T, int E, int k, int32_t* counts, int32_t* offsets,
                int32_t* dst_row, int32_t* src_tok, void* ws, hipStream_t s);
size_t index_ws_bytes(int T, int E);
int local_ids(const int32_t* topk_idx, int n, int e_lo, int e_count, int32_t* out, hipStream_t s);
int fp8_convert_selftest(unsigned long long* mismatches, hipStream_t s);
int permute_rows(const void* src, int src_dt, const int32_t* dst_row, const float* row_scale,
                 int T, int h, int k, void* dst, int dst_dt, float* dst_scale, hipStream_t s);
int combine_rows(const void* yp, int yp_dt, const int32_t* dst_row, const float* w, int T, int h,
                 int k, void* y, int y_dt, hipStream_t s);
int grouped_fwd(const void* xp, const float* xp_scale, const moe_weights* W,
                const int32_t* offsets, int rows, void* h13_save, void* yp, int yp_dtype, void* ws,
                hipStream_t s);
size_t grouped_fwd_ws_bytes(int rows, int h, int h_ffn, int E, int dtype);
int grouped_bwd(const void* dyp, const void* xp, const void* h13_save, const moe_weights* W,
                const int32_t* offsets, int rows, void* dxp, float* dw1, float* dw3, float* dw2,
                void* ws, hipStream_t s);
size_t grouped_bwd_ws_bytes(int rows, int h, int h_ffn, int E, int dtype);
int dw_rows_bf16(const void* a, int M, const void* b, int N, const int32_t* offsets, int E,
                 int rows, float* out, hipStream_t s);
int router_bwd(const void* dy, const void* yp, int yp_dtype, const int32_t* dst_row, const int32_t* topk_idx,
               const float* topk_w, const float* logits, const int32_t* counts, int T, int h,
               int E, int k, float alpha, int dtype, const void* x, const void* w_gate,
               const float* dx_in, void* dx, float* dlogits, float* dw_gate, float* dbias,
               void* ws, hipStream_t s);
size_t router_bwd_ws_bytes(int T, int h, int E);
int router_aux(const float* logits, const int32_t* counts, int T, int E, int k, float alpha,
               float* loss, void* ws, hipStream_t s);
size_t router_aux_ws_bytes(int T, int E);
int capacity_drop(const int32_t* topk_idx, const float* logits, int T, int E, int k, int group,
                  int capacity, int32_t* out, void* ws, hipStream_t s);
size_t capacity_ws_bytes(int T, int E, int k);
int pack_weights(const void* w1, const void* w3, const void* w2, int in_dt, int E, int h,
                 int h_ffn, int out_dt, void* w13, void* w2p, float* w13_scale, float* w2_scale,
                 void* w13_bwd, void* w2_bwd, float* w13_bwd_scale, float* w2_bwd_scale,
                 hipStream_t s);
int grouped_bwd_fp8(const void* dyp_q, const float* dyp_scale, const void* dyp, const void* xp,
                    const void* h13_save, const moe_weights* W, const int32_t* offsets, int rows,
                    void* dxp, float* dw1, float* dw3, float* dw2, void* ws, hipStream_t s,
                    const int32_t* dst_row = nullptr, const float* topk_w = nullptr, int T = 0,
                    int k = 0);
size_t grouped_bwd_fp8_ws_bytes(int rows, int h, int h_ffn, int E);
int dispatch_swiglu_fwd(const void* x, const int32_t* topk_idx, int T, int k, int32_t* counts,
                        int32_t* offsets, int32_t* dst_row, int32_t* src_tok, const moe_weights* W,
                        void* xp, void* h13_save, void* yp, int yp_f32, int32_t* status, void* ws,
                        hipStream_t s, int spin_limit = 1 << 20, bool copy = true);
size_t arrival_ws_bytes(int T, int k, int h, int h_ffn, int E);
int num_cus();

// Launch status: clear_status() before a call's first launch drops any error
// left by earlier HIP calls of other code; launch_status() after the last
// launch returns MOE_OK or MOE_ERR_HIP and keeps the HIP error text.
void clear_status();
int launch_status();
const char* last_hip_error();

// Optional per-kernel timing: when enabled (moe_timing_enable), a pair of HIP
// events is recorded on the launch stream around every kernel of the layer.
// A negative id records nothing (a kernel inside another timed span).
enum TimerId { kTRoute = 0, kTIndex, kTPermute, kTFc1, kTQuant, kTFc2, kTCombine, kTBwd1, kTBwd2,
               kTBwd3, kTBwd4, kTPack, kTXpose, kTRouterBwd, kTRouterAux, kTCapacity, kNumTimers };
void timer_begin(int id, hipStream_t s);
void timer_end(int id, hipStream_t s);
}  // namespace moe_launch
