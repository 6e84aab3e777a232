// Dispatch copy and weighted combine: the two HBM-bound row movers.
//
// Dispatch (local scatter into expert-contiguous rows): MegaScale-MoE paper
// review, §四 adaptive EP communication; research digest §3.3.  Per-token FP8
// scales on the dispatched rows: review §三 communication-compression layer
// and §四 FP8 row; digest §3.4.  Combine (weighted sum of a token's expert
// outputs): review §三 training flow "token aggregation"; DisagMoE page §2.1.
//
// Each lane moves 16-byte chunks, so a wave moves 1 KB per instruction; the
// token row is read once and written k times (dispatch), or the k routed rows
// are read once and one row written (combine), which is the minimum HBM
// traffic of either step.
#include "common.h"

namespace moe {

constexpr int kRowsPerBlock = 4;  // waves per 256-thread block

// 8 bf16 values from 16 bytes.
__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[i]); f[2 * i + 1] = bf16_hi(v[i]); }
}

// One wavefront per token: the row is loaded in batches of chunks and each
// batch is stored to the token's k routed rows.
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
  constexpr int kBatch = 8;          // chunks per lane in flight
  const int nch = h / EPC;
  const u32x4* s = reinterpret_cast<const u32x4*>(static_cast<const char*>(src) + size_t(t) * h * (16 / EPC));
  for (int c0 = lane; c0 < nch; c0 += 64 * kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (c0 + 64 * b < nch) v[b] = s[c0 + 64 * b];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + 64 * b;
      if (c >= nch) break;
      for (int j = 0; j < k; ++j) {
        if (rows[j] < 0 || rows[j] >= T * k) continue;
        u32x4 o = v[b];
        if (row_scale) {
          if (kF32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(__uint_as_float(o[i]) * sc[j]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              o[i] = pack_bf16x2(bf16_lo(o[i]) * sc[j], bf16_hi(o[i]) * sc[j]);
          }
        }
        reinterpret_cast<u32x4*>(static_cast<char*>(dst) + size_t(rows[j]) * h * (16 / EPC))[c] = o;
      }
    }
  }
}

// One thread per 16-byte chunk of a token row: the chunk is loaded once and
// stored to each of the token's k routed rows.
template <bool kF32, bool kNTL, bool kNTS>
__global__ void __launch_bounds__(256) permute_flat_kernel(const void* __restrict__ src,
                                                           const int32_t* __restrict__ dst_row,
                                                           const float* __restrict__ row_scale,
                                                           int T, int h, int k,
                                                           void* __restrict__ dst) {
  constexpr int EPC = kF32 ? 4 : 8;  // elements per 16-byte chunk
  const int nch = h / EPC;
  const size_t gid = size_t(blockIdx.x) * 256 + threadIdx.x;
  const int t = int(gid / unsigned(nch));
  const int c = int(gid - size_t(t) * nch);
  if (t >= T) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(static_cast<const char*>(src) + size_t(t) * h * (16 / EPC)) + c;
  const u32x4 v = kNTL ? __builtin_nontemporal_load(s) : *s;
  for (int j = 0; j < k; ++j) {
    const int r = dst_row[size_t(t) * k + j];
    if (r < 0 || r >= T * k) continue;
    u32x4 o = v;
    if (row_scale) {
      const float sc = row_scale[size_t(t) * k + j];
      if (kF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(__uint_as_float(o[i]) * sc);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(bf16_lo(o[i]) * sc, bf16_hi(o[i]) * sc);
      }
    }
    u32x4* d = reinterpret_cast<u32x4*>(static_cast<char*>(dst) + size_t(r) * h * (16 / EPC)) + c;
    if (kNTS) __builtin_nontemporal_store(o, d); else *d = o;
  }
}

// BF16 rows -> per-token E4M3 codes + scale (amax / 448) on every routed copy.
// With row_scale, routed row (t, j) keeps the codes of src[t] and its scale
// becomes row_scale[t][j] * scale_t.
__global__ void __launch_bounds__(256) permute_fp8_kernel(const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst_row,
                                                          const float* __restrict__ row_scale,
                                                          int T, int h, int k,
                                                          uint8_t* __restrict__ dst,
                                                          float* __restrict__ dst_scale) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nch = h / 8;
  constexpr int kBatch = 16;  // chunks per lane in flight (h <= 8192: the whole row)
  const u32x4* s = reinterpret_cast<const u32x4*>(src + size_t(t) * h);
  int rows[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) rows[j] = dst_row[size_t(t) * k + j];
  u32x4 v[kBatch];
  float amax = 0.f;
  for (int c0 = lane; c0 < nch; c0 += 64 * kBatch) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) v[b] = c0 + 64 * b < nch ? s[c0 + 64 * b] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      float f[8];
      unpack8(v[b], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    }
  }
  amax = wave_max(amax);
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  if (lane < k && rows[lane] >= 0 && rows[lane] < T * k)
    dst_scale[rows[lane]] = row_scale ? row_scale[size_t(t) * k + lane] * scale : scale;
  const QuotScale qs = quot_scale(scale);
  const bool held = nch <= 64 * kBatch;  // v still holds the row
  for (int c0 = lane; c0 < nch; c0 += 64 * kBatch) {
    if (!held) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (c0 + 64 * b < nch) v[b] = s[c0 + 64 * b];
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + 64 * b;
      if (c >= nch) break;
      float f[8];
      unpack8(v[b], f);
      const uint32_t lo = e4m3x4_quot(f[0], f[1], f[2], f[3], qs);
      const uint32_t hi = e4m3x4_quot(f[4], f[5], f[6], f[7], qs);
      for (int j = 0; j < k; ++j) {
        if (rows[j] < 0 || rows[j] >= T * k) continue;
        uint2* d = reinterpret_cast<uint2*>(dst + size_t(rows[j]) * h);
        d[c] = make_uint2(lo, hi);
      }
    }
  }
}

// KM >= k bounds the routed rows per token, so every load of a chunk
// position is issued before the first add.  WPT waves share a token, each
// taking a contiguous slice of the row; kNTL / kNTS make the loads / stores
// nontemporal (the rows are touched once).
template <bool kInF32, bool kOutF32, int KM, bool kNTL, bool kNTS, int WPT>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ yp,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ w, int T, int h,
                                                      int k, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wv = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int t = wv / WPT, part = wv - t * WPT;
  if (t >= T) return;
  int rows[KM];
  float wt[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    rows[j] = -1;
    wt[j] = 0.f;
    if (j < k) {
      const int r = dst_row[size_t(t) * k + j];
      rows[j] = (r < 0 || r >= T * k) ? -1 : r;
      wt[j] = w ? w[size_t(t) * k + j] : 1.f;
    }
  }
  constexpr int kBatch = KM <= 2 ? 8 : (16 / KM > 0 ? 16 / KM : 1);  // ~16 loads in flight
  constexpr int kVec = kInF32 ? 2 : 1;     // 16-byte loads per 8 elements
  const int nch = h / 8 / WPT;   // 8-element chunks of this wave's slice
  const int cb = part * nch;
  for (int c0 = lane; c0 < nch; c0 += 64 * kBatch) {
    u32x4 v[kBatch][KM][kVec];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
#pragma unroll
      for (int j = 0; j < KM; ++j)
#pragma unroll
        for (int q = 0; q < kVec; ++q) {
          v[b][j][q] = u32x4{0, 0, 0, 0};
          const int c = c0 + 64 * b;
          if (rows[j] >= 0 && c < nch) {
            const char* base = static_cast<const char*>(yp) + size_t(rows[j]) * h * (kInF32 ? 4 : 2);
            const u32x4* p = reinterpret_cast<const u32x4*>(base) + (cb + c) * kVec + q;
            v[b][j][q] = kNTL ? __builtin_nontemporal_load(p) : *p;
          }
        }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + 64 * b;
      if (c >= nch) break;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (rows[j] < 0) continue;
        float f[8];
        if (kInF32) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[i] = __uint_as_float(v[b][j][0][i]);
            f[4 + i] = __uint_as_float(v[b][j][kVec - 1][i]);
          }
        } else {
          unpack8(v[b][j][0], f);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], f[i], acc[i]);
      }
      if (kOutF32) {
        f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(y) + size_t(t) * h + (cb + c) * 8);
        const f32x4 o0{acc[0], acc[1], acc[2], acc[3]}, o1{acc[4], acc[5], acc[6], acc[7]};
        if (kNTS) { __builtin_nontemporal_store(o0, p); __builtin_nontemporal_store(o1, p + 1); }
        else { p[0] = o0; p[1] = o1; }
      } else {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        u32x4* p = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + size_t(t) * h) + cb + c;
        if (kNTS) __builtin_nontemporal_store(o, p); else *p = o;
      }
    }
  }
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

// Dispatch copy: for k <= 4 one thread per 16-byte chunk with nontemporal
// loads and stores (measured in the layer: Mixtral-shaped, k = 2, 0.74 -> 0.78
// of HBM peak; 352B-shaped, k = 3, 0.70 -> 0.79); for larger k the
// wave-per-token kernel, whose k stores per loaded chunk measured faster there
// (DeepSeekMoE-shaped, k = 6: 0.71 against 0.68).
int permute_rows(const void* src, int src_dt, const int32_t* dst_row, const float* row_scale,
                 int T, int h, int k, void* dst, int dst_dt, float* dst_scale, hipStream_t s) {
  if (T == 0) return MOE_OK;
  dim3 grid(ceil_div(T, kRowsPerBlock)), block(256);
  const bool f32 = src_dt == MOE_F32;
  const dim3 fgrid(unsigned((size_t(T) * (h / (f32 ? 4 : 8)) + 255) / 256));
  timer_begin(kTPermute, s);
  if (dst_dt == MOE_FP8_E4M3) {
    hipLaunchKernelGGL(permute_fp8_kernel, grid, block, 0, s, (const uint16_t*)src, dst_row, row_scale,
                       T, h, k, (uint8_t*)dst, dst_scale);
  } else if (k <= 4) {
    if (f32)
      hipLaunchKernelGGL((permute_flat_kernel<true, true, true>), fgrid, block, 0, s, src, dst_row,
                         row_scale, T, h, k, dst);
    else
      hipLaunchKernelGGL((permute_flat_kernel<false, true, true>), fgrid, block, 0, s, src, dst_row,
                         row_scale, T, h, k, dst);
  } else if (f32) {
    hipLaunchKernelGGL(permute_copy_kernel<true>, grid, block, 0, s, src, dst_row, row_scale, T, h,
                       k, dst);
  } else {
    hipLaunchKernelGGL(permute_copy_kernel<false>, grid, block, 0, s, src, dst_row, row_scale, T,
                       h, k, dst);
  }
  timer_end(kTPermute, s);
  return launch_status();
}

template <bool in32, bool out32, int WPT>
static void launch_combine_w(const void* yp, const int32_t* dst_row, const float* w, int T, int h,
                             int k, void* y, hipStream_t s) {
  const dim3 grid(ceil_div(T * WPT, kRowsPerBlock)), block(256);
  if (k <= 1)
    hipLaunchKernelGGL((combine_kernel<in32, out32, 1, true, true, WPT>), grid, block, 0, s, yp,
                       dst_row, w, T, h, k, y);
  else if (k <= 2)
    hipLaunchKernelGGL((combine_kernel<in32, out32, 2, true, true, WPT>), grid, block, 0, s, yp,
                       dst_row, w, T, h, k, y);
  else if (k <= 4)
    hipLaunchKernelGGL((combine_kernel<in32, out32, 4, true, true, WPT>), grid, block, 0, s, yp,
                       dst_row, w, T, h, k, y);
  else if (k <= 8)
    hipLaunchKernelGGL((combine_kernel<in32, out32, 8, true, true, WPT>), grid, block, 0, s, yp,
                       dst_row, w, T, h, k, y);
  else
    hipLaunchKernelGGL((combine_kernel<in32, out32, MOE_MAX_TOPK, true, true, WPT>), grid, block, 0,
                       s, yp, dst_row, w, T, h, k, y);
}

// Combine: two waves per token (each half of the row) with nontemporal loads
// and stores; measured in the layer, 0.65 -> 0.71 of HBM peak (Mixtral-shaped)
// and 0.53 -> 0.66 (DeepSeekMoE-shaped, k = 6).  A row of an odd number of
// 8-element chunks stays on one wave.
template <bool in32, bool out32>
static void launch_combine(const void* yp, const int32_t* dst_row, const float* w, int T, int h,
                           int k, void* y, hipStream_t s) {
  if ((h / 8) % 2 == 0) launch_combine_w<in32, out32, 2>(yp, dst_row, w, T, h, k, y, s);
  else launch_combine_w<in32, out32, 1>(yp, dst_row, w, T, h, k, y, s);
}

int combine_rows(const void* yp, int yp_dt, const int32_t* dst_row, const float* w, int T, int h,
                 int k, void* y, int y_dt, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const bool in32 = yp_dt == MOE_F32, out32 = y_dt == MOE_F32;
  timer_begin(kTCombine, s);
  if (in32 && out32) launch_combine<true, true>(yp, dst_row, w, T, h, k, y, s);
  else if (in32) launch_combine<true, false>(yp, dst_row, w, T, h, k, y, s);
  else if (out32) launch_combine<false, true>(yp, dst_row, w, T, h, k, y, s);
  else launch_combine<false, false>(yp, dst_row, w, T, h, k, y, s);
  timer_end(kTCombine, s);
  return launch_status();
}

}  // namespace moe_launch
