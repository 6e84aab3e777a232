// Router: gate GEMM + top-k + softmax over the selected logits.
//
// Gate scores and top-k selection: MegaScale-MoE paper review, §三 (MoE
// layer structure, Fig. 2; training flow "token routing"); DisagMoE page,
// §2.1 / Fig. 2(a) (k highest-scoring experts, weighted sum).  Softmax over
// the k kept logits and the tie rule (lower expert index first) are this
// library's reading of the unspecified details.
//
// One workgroup of 256 threads handles 128 tokens.  BF16: the logits come
// from MFMA 32x32x16 (each wave 32 tokens x all experts), reading x straight
// from HBM in 16-byte loads and the gate weight through LDS in K slabs,
// transposed so both operands are K-contiguous.  The 128 x E fp32 logits then
// go to LDS and one thread per token selects its k experts.
#include "common.h"

namespace moe {

constexpr int kRouteTokens = 128;
constexpr int kRouteSlab = 64;  // K elements per LDS slab

// LDS slab for W_g^T: [E_pad][kRouteSlab + 8] bf16 (row padded by 16 B).
constexpr int kSlabStride = kRouteSlab + 8;

__device__ __forceinline__ void topk_select(const float* L, int E, int k, int32_t* idx_out,
                                            float* w_out) {
  // j-th pick = the largest logit strictly after the previous pick in the
  // (logit desc, index asc) order.
  float pv = 0.f;
  int pe = -1;
  float vals[MOE_MAX_TOPK];
  int ids[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int be = -1;
    for (int e = 0; e < E; ++e) {
      float v = L[e];
      bool after = pe < 0 || v < pv || (v == pv && e > pe);
      if (after && (be < 0 || v > bv)) { bv = v; be = e; }
    }
    vals[j] = bv; ids[j] = be;
    pv = bv; pe = be;
  }
  float z[MOE_MAX_TOPK];
  float s = 0.f;
  for (int j = 0; j < k; ++j) { z[j] = expf(vals[j] - vals[0]); s += z[j]; }
  float inv = 1.0f / s;
  for (int j = 0; j < k; ++j) {
    idx_out[j] = ids[j];
    w_out[j] = (k == 1) ? 1.0f : z[j] * inv;
  }
}

template <int NT>  // NT = ceil(E / 32) expert tiles of 32
__global__ void __launch_bounds__(256) route_bf16_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wg,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits_out, int T,
                                                         int h, int E, int k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* slab = reinterpret_cast<uint16_t*>(smem);  // [NT*32][kSlabStride]
  float* lg = reinterpret_cast<float*>(smem);          // [128][E+1] after the GEMM

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRouteTokens;
  const int row = t0 + wave * 32 + (lane & 31);
  const int half = lane >> 5;
  const int rowc = row < T ? row : T - 1;
  const uint16_t* xr = x + size_t(rowc) * h + half * 32;

  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;

  const int Ep = NT * 32;
  for (int k0 = 0; k0 < h; k0 += kRouteSlab) {
    // x: 64 contiguous bytes per lane (4 x 16 B) at k0 + 32*half.
    u32x4 xa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xa[s] = *reinterpret_cast<const u32x4*>(xr + k0 + s * 8);
    __syncthreads();  // previous slab fully consumed
    for (int q = tid; q < kRouteSlab * Ep; q += 256) {
      int kk = q / Ep, e = q - kk * Ep;
      uint16_t v = e < E ? wg[size_t(k0 + kk) * E + e] : uint16_t(0);
      slab[e * kSlabStride + kk] = v;
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint16_t* br = slab + (n * 32 + (lane & 31)) * kSlabStride + half * 32;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 b = *reinterpret_cast<const u32x4*>(br + s * 8);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, xa[s]), __builtin_bit_cast(bf16x8, b), acc[n], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  const int ls = E + 1;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    int e = n * 32 + (lane & 31);
    if (e < E) {
      float b = bias ? bias[e] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int i = wave * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        lg[i * ls + e] = acc[n][r] + b;
      }
    }
  }
  __syncthreads();
  if (logits_out) {
    for (int q = tid; q < kRouteTokens * E; q += 256) {
      int i = q / E, e = q - i * E;
      if (t0 + i < T) logits_out[size_t(t0 + i) * E + e] = lg[i * ls + e];
    }
  }
  if (tid < kRouteTokens && t0 + tid < T) {
    int t = t0 + tid;
    topk_select(lg + tid * ls, E, k, topk_idx + size_t(t) * k, topk_w + size_t(t) * k);
  }
}

// FP32 inputs, or logits given: plain dot products (small workloads only).
__global__ void __launch_bounds__(256) route_generic_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ wg,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T,
                                                            int h, int E, int k,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* lg = reinterpret_cast<float*>(smem);
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRouteTokens;
  const int ls = E + 1;
  for (int q = tid; q < kRouteTokens * E; q += 256) {
    int i = q / E, e = q - i * E;
    int t = t0 + i;
    float v = 0.f;
    if (t < T) {
      if (x) {
        const float* xr = x + size_t(t) * h;
        for (int c = 0; c < h; ++c) v = fmaf(xr[c], wg[size_t(c) * E + e], v);
        if (bias) v += bias[e];
        if (logits) logits[size_t(t) * E + e] = v;
      } else {
        v = logits[size_t(t) * E + e];
      }
    }
    lg[i * ls + e] = v;
  }
  __syncthreads();
  if (tid < kRouteTokens && t0 + tid < T) {
    int t = t0 + tid;
    topk_select(lg + tid * ls, E, k, topk_idx + size_t(t) * k, topk_w + size_t(t) * k);
  }
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

template <int NT>
static void launch_route_bf16(const void* x, const void* wg, const float* bias, float* logits,
                              int T, int h, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  size_t slab = size_t(NT * 32) * kSlabStride * 2;
  size_t lgb = size_t(kRouteTokens) * (E + 1) * 4;
  size_t shm = slab > lgb ? slab : lgb;
  static bool ok = allow_lds(route_bf16_kernel<NT>, 160 * 1024);
  (void)ok;
  hipLaunchKernelGGL(route_bf16_kernel<NT>, dim3(ceil_div(T, kRouteTokens)), dim3(256), shm, s,
                     (const uint16_t*)x, (const uint16_t*)wg, bias, logits, T, h, E, k, idx, w);
}

int route(const void* x, const void* w_gate, const float* bias, float* logits, int T, int h,
          int E, int k, int dtype, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (T == 0) return MOE_OK;
  timer_begin(kTRoute, s);
  if (x && dtype == MOE_BF16) {
    int nt = ceil_div(E, 32);
    switch (nt) {
      case 1: launch_route_bf16<1>(x, w_gate, bias, logits, T, h, E, k, topk_idx, topk_w, s); break;
      case 2: launch_route_bf16<2>(x, w_gate, bias, logits, T, h, E, k, topk_idx, topk_w, s); break;
      case 3: launch_route_bf16<3>(x, w_gate, bias, logits, T, h, E, k, topk_idx, topk_w, s); break;
      case 4: launch_route_bf16<4>(x, w_gate, bias, logits, T, h, E, k, topk_idx, topk_w, s); break;
      case 5: launch_route_bf16<5>(x, w_gate, bias, logits, T, h, E, k, topk_idx, topk_w, s); break;
      case 6: launch_route_bf16<6>(x, w_gate, bias, logits, T, h, E, k, topk_idx, topk_w, s); break;
      case 7: launch_route_bf16<7>(x, w_gate, bias, logits, T, h, E, k, topk_idx, topk_w, s); break;
      default: launch_route_bf16<8>(x, w_gate, bias, logits, T, h, E, k, topk_idx, topk_w, s); break;
    }
  } else {
    size_t shm = size_t(kRouteTokens) * (E + 1) * 4;
    static bool ok = allow_lds(route_generic_kernel, 160 * 1024);
    (void)ok;
    hipLaunchKernelGGL(route_generic_kernel, dim3(ceil_div(T, kRouteTokens)), dim3(256), shm, s,
                       (const float*)x, (const float*)w_gate, x ? bias : nullptr, logits, T, h, E,
                       k, topk_idx, topk_w);
  }
  timer_end(kTRoute, s);
  return launch_status();
}

}  // namespace moe_launch
