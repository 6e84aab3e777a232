// Dispatch copy and weighted combine: the two HBM-bound row movers.
//
// Dispatch (local scatter into expert-contiguous rows): MegaScale-MoE paper
// review, §四 adaptive EP communication; research digest §3.3.  Per-token FP8
// scales on the dispatched rows: review §三 communication-compression layer
// and §四 FP8 row; digest §3.4.  Combine (weighted sum of a token's expert
// outputs): review §三 training flow "token aggregation"; DisagMoE page §2.1.
//
// One wavefront per token.  Each lane moves 16-byte chunks, so a wave moves
// 1 KB per instruction; the token row is read once and written k times
// (dispatch), or the k routed rows are read once and one row written
// (combine), which is the minimum HBM traffic of either step.
#include "common.h"

namespace moe {

constexpr int kRowsPerBlock = 4;  // tokens (waves) per 256-thread block

// 8 bf16 values from 16 bytes.
__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[i]); f[2 * i + 1] = bf16_hi(v[i]); }
}

template <bool kF32>
__global__ void __launch_bounds__(256) permute_copy_kernel(const void* __restrict__ src,
                                                           const int32_t* __restrict__ dst_row,
                                                           const float* __restrict__ row_scale,
                                                           int T, int h, int k,
                                                           void* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[MOE_MAX_TOPK];
  float sc[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    rows[j] = dst_row[size_t(t) * k + j];
    sc[j] = row_scale ? row_scale[size_t(t) * k + j] : 1.f;
  }
  constexpr int EPC = kF32 ? 4 : 8;  // elements per 16-byte chunk
  const int nch = h / EPC;
  const u32x4* s = reinterpret_cast<const u32x4*>(static_cast<const char*>(src) + size_t(t) * h * (16 / EPC));
  for (int c = lane; c < nch; c += 64) {
    u32x4 v = s[c];
    for (int j = 0; j < k; ++j) {
      if (rows[j] < 0 || rows[j] >= T * k) continue;
      u32x4 o = v;
      if (row_scale) {
        if (kF32) {
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(__uint_as_float(v[i]) * sc[j]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[i] = pack_bf16x2(bf16_lo(v[i]) * sc[j], bf16_hi(v[i]) * sc[j]);
        }
      }
      reinterpret_cast<u32x4*>(static_cast<char*>(dst) + size_t(rows[j]) * h * (16 / EPC))[c] = o;
    }
  }
}

// BF16 rows -> per-token E4M3 codes + scale (amax / 448) on every routed copy.
__global__ void __launch_bounds__(256) permute_fp8_kernel(const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst_row,
                                                          int T, int h, int k,
                                                          uint8_t* __restrict__ dst,
                                                          float* __restrict__ dst_scale) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nch = h / 8;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + size_t(t) * h);
  float amax = 0.f;
  for (int c = lane; c < nch; c += 64) {
    u32x4 v = s[c];
    float f[8];
    unpack8(v, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = wave_max(amax);
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  int rows[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) rows[j] = dst_row[size_t(t) * k + j];
  if (lane < k && rows[lane] >= 0 && rows[lane] < T * k) dst_scale[rows[lane]] = scale;
  for (int c = lane; c < nch; c += 64) {
    u32x4 v = s[c];
    float f[8];
    unpack8(v, f);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(f[i] / scale) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(f[4 + i] / scale) << (8 * i);
    for (int j = 0; j < k; ++j) {
      if (rows[j] < 0 || rows[j] >= T * k) continue;
      uint2* d = reinterpret_cast<uint2*>(dst + size_t(rows[j]) * h);
      d[c] = make_uint2(lo, hi);
    }
  }
}

template <bool kInF32, bool kOutF32>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ yp,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ w, int T, int h,
                                                      int k, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[MOE_MAX_TOPK];
  float wt[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    rows[j] = dst_row[size_t(t) * k + j];
    wt[j] = w ? w[size_t(t) * k + j] : 1.f;
  }
  const int nch = h / 8;  // 8 elements per step (two 16-byte chunks for fp32)
  for (int c = lane; c < nch; c += 64) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      if (rows[j] < 0 || rows[j] >= T * k) continue;
      float f[8];
      if (kInF32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(yp) + size_t(rows[j]) * h + c * 8);
        f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
      } else {
        u32x4 v = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(yp) + size_t(rows[j]) * h)[c];
        unpack8(v, f);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], f[i], acc[i]);
    }
    if (kOutF32) {
      f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(y) + size_t(t) * h + c * 8);
      p[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      p[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + size_t(t) * h)[c] = o;
    }
  }
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

int permute_rows(const void* src, int src_dt, const int32_t* dst_row, const float* row_scale,
                 int T, int h, int k, void* dst, int dst_dt, float* dst_scale, hipStream_t s) {
  if (T == 0) return MOE_OK;
  dim3 grid(ceil_div(T, kRowsPerBlock)), block(256);
  timer_begin(kTPermute, s);
  if (dst_dt == MOE_FP8_E4M3) {
    hipLaunchKernelGGL(permute_fp8_kernel, grid, block, 0, s, (const uint16_t*)src, dst_row, T, h,
                       k, (uint8_t*)dst, dst_scale);
  } else if (src_dt == MOE_F32) {
    hipLaunchKernelGGL(permute_copy_kernel<true>, grid, block, 0, s, src, dst_row, row_scale, T, h,
                       k, dst);
  } else {
    hipLaunchKernelGGL(permute_copy_kernel<false>, grid, block, 0, s, src, dst_row, row_scale, T,
                       h, k, dst);
  }
  timer_end(kTPermute, s);
  return launch_status();
}

int combine_rows(const void* yp, int yp_dt, const int32_t* dst_row, const float* w, int T, int h,
                 int k, void* y, int y_dt, hipStream_t s) {
  if (T == 0) return MOE_OK;
  dim3 grid(ceil_div(T, kRowsPerBlock)), block(256);
  bool in32 = yp_dt == MOE_F32, out32 = y_dt == MOE_F32;
  timer_begin(kTCombine, s);
  if (in32 && out32)
    hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, s, yp, dst_row, w, T, h, k, y);
  else if (in32)
    hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, s, yp, dst_row, w, T, h, k, y);
  else if (out32)
    hipLaunchKernelGGL((combine_kernel<false, true>), grid, block, 0, s, yp, dst_row, w, T, h, k, y);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, s, yp, dst_row, w, T, h, k, y);
  timer_end(kTCombine, s);
  return launch_status();
}

}  // namespace moe_launch
