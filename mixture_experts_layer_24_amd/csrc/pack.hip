// Weight packing (set-up, outside the per-step path).
//
// Expert weights arrive as W1, W3 [E][h][h_ffn] and W2 [E][h_ffn][h] (y = x W).
// The GroupedGEMM wants both operands K-contiguous, so each matrix is stored
// transposed; FC1's gate and up projections are interleaved in blocks of 32
// output channels so one tile produces matching gate/up pairs.  For FP8 each
// output channel gets its own scale amax/448 over the input dimension (the
// per-channel weight counterpart of the per-token activation scales of the
// MegaScale-MoE paper review, §三 compression layer and §四 FP8 row).
#include "common.h"

namespace moe {

enum { kMapIdentity = 0, kMapGate = 1, kMapUp = 2 };

__device__ __forceinline__ int map_col(int c, int mode) {
  if (mode == kMapIdentity) return c;
  return (c >> 5) * 64 + (mode == kMapUp ? 32 : 0) + (c & 31);
}

template <bool kInF32>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if (kInF32) return static_cast<const float*>(p)[i];
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Per-output-channel scale: one thread per (expert, source column).
template <bool kInF32>
__global__ void col_scale_kernel(const void* __restrict__ src, int rows_s, int cols_s,
                                 float* __restrict__ scale, int ld_scale, int mode) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int e = blockIdx.y;
  if (c >= cols_s) return;
  const size_t base = size_t(e) * rows_s * cols_s;
  float amax = 0.f;
  for (int r = 0; r < rows_s; ++r) amax = fmaxf(amax, fabsf(load_elem<kInF32>(src, base + size_t(r) * cols_s + c)));
  scale[size_t(e) * ld_scale + map_col(c, mode)] = amax > 0.f ? amax / 448.0f : 1.0f;
}

// dst[e][map(c)][r] = convert(src[e][r][c]); 32 x 32 tiles through LDS.
template <bool kInF32, int OUT>
__global__ void __launch_bounds__(256) transpose_kernel(const void* __restrict__ src, int rows_s,
                                                        int cols_s, void* __restrict__ dst,
                                                        int dst_rows, const float* __restrict__ scale,
                                                        int ld_scale, int mode) {
  __shared__ float tile[32][33];
  const int e = blockIdx.z;
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const size_t sbase = size_t(e) * rows_s * cols_s;
  for (int i = ty; i < 32; i += 8)
    tile[i][tx] = load_elem<kInF32>(src, sbase + size_t(r0 + i) * cols_s + c0 + tx);
  __syncthreads();
  const size_t dbase = size_t(e) * dst_rows * rows_s;
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i;                 // source column -> destination row
    const int p = map_col(c, mode);
    const float v = tile[tx][i];
    const size_t o = dbase + size_t(p) * rows_s + r0 + tx;
    if (OUT == MOE_F32) {
      static_cast<float*>(dst)[o] = v;
    } else if (OUT == MOE_BF16) {
      static_cast<uint16_t*>(dst)[o] = uint16_t(f32_to_bf16_bits(v));
    } else {
      const float s = scale[size_t(e) * ld_scale + p];
      static_cast<uint8_t*>(dst)[o] = uint8_t(f32_to_e4m3(v / s));
    }
  }
}

// Backward layout of W1 | W3: dst[e][i][p] = (p/32 odd ? W3 : W1)[e][i][(p/64)*32 + p%32],
// 16 bytes (8 bf16) per thread.
__global__ void interleave13_kernel(const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3,
                                    int E, int h, int hf, uint16_t* __restrict__ dst) {
  const size_t q = size_t(blockIdx.x) * blockDim.x + threadIdx.x;  // 8-element chunk of dst
  const size_t per_row = size_t(2 * hf) / 8;
  const size_t total = size_t(E) * h * per_row;
  if (q >= total) return;
  const size_t row = q / per_row;                  // e * h + i
  const int p = int(q - row * per_row) * 8;
  const int ch = (p >> 6) * 32 + (p & 31);
  const uint16_t* src = ((p >> 5) & 1) ? w3 : w1;
  *reinterpret_cast<u32x4*>(dst + row * (2 * hf) + p) =
      *reinterpret_cast<const u32x4*>(src + row * hf + ch);
}

// FP8 backward copies: one scale per row over the contracted dimension.
// w2_bwd rows are W2's rows (h_ffn channels over h); w13_bwd row i of expert e
// interleaves W1[e][i][:] and W3[e][i][:] like interleave13_kernel, one scale
// over both.  One wave per row.
__global__ void __launch_bounds__(256) rowq_w2_kernel(const uint16_t* __restrict__ w2, int n, int h,
                                                      uint8_t* __restrict__ dst,
                                                      float* __restrict__ scale) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  rowq_wave(w2 + size_t(r) * h, h, dst + size_t(r) * h, scale + r);
}

__global__ void __launch_bounds__(256) rowq_w13_kernel(const uint16_t* __restrict__ w1,
                                                       const uint16_t* __restrict__ w3, int n,
                                                       int hf, uint8_t* __restrict__ dst,
                                                       float* __restrict__ scale) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);  // r = e * h + i
  if (r >= n) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* a = w1 + size_t(r) * hf;
  const uint16_t* b = w3 + size_t(r) * hf;
  float amax = 0.f;
  for (int c = lane * 8; c < hf; c += 512) {
    const u32x4 va = *reinterpret_cast<const u32x4*>(a + c), vb = *reinterpret_cast<const u32x4*>(b + c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_lo(va[i])), fabsf(bf16_hi(va[i]))),
                               fmaxf(fabsf(bf16_lo(vb[i])), fabsf(bf16_hi(vb[i])))));
  }
  amax = wave_max(amax);
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (lane == 0) scale[r] = s;
  uint8_t* d = dst + size_t(r) * 2 * hf;
  for (int p = lane * 8; p < 2 * hf; p += 512) {
    const int ch = (p >> 6) * 32 + (p & 31);
    const u32x4 v = *reinterpret_cast<const u32x4*>((((p >> 5) & 1) ? b : a) + ch);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo |= f32_to_e4m3(bf16_lo(v[i]) / s) << (16 * i);
      lo |= f32_to_e4m3(bf16_hi(v[i]) / s) << (16 * i + 8);
      hi |= f32_to_e4m3(bf16_lo(v[2 + i]) / s) << (16 * i);
      hi |= f32_to_e4m3(bf16_hi(v[2 + i]) / s) << (16 * i + 8);
    }
    *reinterpret_cast<uint2*>(d + p) = make_uint2(lo, hi);
  }
}

__global__ void copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t q = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q < n) dst[q] = src[q];
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

template <bool kInF32, int OUT>
static void pack_one(const void* src, int E, int rows_s, int cols_s, void* dst, int dst_rows,
                     float* scale, int ld_scale, int mode, hipStream_t s) {
  if (OUT == MOE_FP8_E4M3)
    hipLaunchKernelGGL(col_scale_kernel<kInF32>, dim3(ceil_div(cols_s, 256), E), dim3(256), 0, s,
                       src, rows_s, cols_s, scale, ld_scale, mode);
  hipLaunchKernelGGL((transpose_kernel<kInF32, OUT>), dim3(cols_s / 32, rows_s / 32, E), dim3(256),
                     0, s, src, rows_s, cols_s, dst, dst_rows, scale, ld_scale, mode);
}

template <bool kInF32, int OUT>
static void pack_all(const void* w1, const void* w3, const void* w2, int E, int h, int hf,
                     void* w13, void* w2p, float* s13, float* s2, hipStream_t s) {
  pack_one<kInF32, OUT>(w1, E, h, hf, w13, 2 * hf, s13, 2 * hf, kMapGate, s);
  pack_one<kInF32, OUT>(w3, E, h, hf, w13, 2 * hf, s13, 2 * hf, kMapUp, s);
  pack_one<kInF32, OUT>(w2, E, hf, h, w2p, h, s2, h, kMapIdentity, s);
}

int pack_weights(const void* w1, const void* w3, const void* w2, int in_dt, int E, int h,
                 int h_ffn, int out_dt, void* w13, void* w2p, float* w13_scale, float* w2_scale,
                 void* w13_bwd, void* w2_bwd, float* w13_bwd_scale, float* w2_bwd_scale,
                 hipStream_t s) {
  timer_begin(kTPack, s);
  if (in_dt == MOE_F32 && out_dt == MOE_F32)
    pack_all<true, MOE_F32>(w1, w3, w2, E, h, h_ffn, w13, w2p, nullptr, nullptr, s);
  else if (in_dt == MOE_BF16 && out_dt == MOE_BF16)
    pack_all<false, MOE_BF16>(w1, w3, w2, E, h, h_ffn, w13, w2p, nullptr, nullptr, s);
  else if (in_dt == MOE_BF16 && out_dt == MOE_FP8_E4M3)
    pack_all<false, MOE_FP8_E4M3>(w1, w3, w2, E, h, h_ffn, w13, w2p, w13_scale, w2_scale, s);
  else
    return MOE_ERR_DTYPE;
  if (out_dt == MOE_FP8_E4M3) {
    if (w13_bwd)
      hipLaunchKernelGGL(rowq_w13_kernel, dim3(ceil_div(E * h, 4)), dim3(256), 0, s, (const uint16_t*)w1,
                         (const uint16_t*)w3, E * h, h_ffn, (uint8_t*)w13_bwd, w13_bwd_scale);
    if (w2_bwd)
      hipLaunchKernelGGL(rowq_w2_kernel, dim3(ceil_div(E * h_ffn, 4)), dim3(256), 0, s, (const uint16_t*)w2,
                         E * h_ffn, h, (uint8_t*)w2_bwd, w2_bwd_scale);
  } else if (w13_bwd) {
    const size_t chunks = size_t(E) * h * (2 * size_t(h_ffn) / 8);
    hipLaunchKernelGGL(interleave13_kernel, dim3(unsigned((chunks + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)w1, (const uint16_t*)w3, E, h, h_ffn, (uint16_t*)w13_bwd);
  }
  if (w2_bwd && out_dt != MOE_FP8_E4M3) {
    const size_t n = size_t(E) * h_ffn * h * 2 / 16;
    hipLaunchKernelGGL(copy16_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s,
                       (const u32x4*)w2, (u32x4*)w2_bwd, n);
  }
  timer_end(kTPack, s);
  return launch_status();
}

}  // namespace moe_launch
