// Token dropping by affinity, per group of experts.
//
// MegaScale-MoE research digest §3.2 (the discussion of Figure 7): load
// balance also drops tokens on each GPU, following DeepSeek-V2, which drops on each
// device the tokens with the lowest affinity until the device's budget is
// met.  A device is a group of `group` consecutive experts (one GPU's share;
// group = 1 is a per-expert capacity): among the (token, slot) pairs routed
// into a group, the `capacity` pairs with the highest affinity
// s = softmax(L_t)[e] over all E experts are kept, equal affinities in
// dispatch order (expert, then token); the others get id -1, which the
// dispatch drops.
//
// Kernels: the index of the full routing (the existing builder); per-token
// softmax statistics; per-row affinity keys (fp32 bits, which order like the
// values since affinities are >= 0); one workgroup per group runs a 4-pass
// radix select for the capacity-th largest key and keeps the ties in row
// order with a block scan.  Every decision is order-independent or taken in
// row order, so the result is deterministic.
#include "common.h"

namespace moe {

// m_t = max_e L[t][e], z_t = sum_e exp(L[t][e] - m_t)
__global__ void __launch_bounds__(256) cap_stats_kernel(const float* __restrict__ logits, int T,
                                                        int E, float2* __restrict__ mz) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* L = logits + size_t(t) * E;
  float m = -INFINITY;
  for (int e = 0; e < E; ++e) m = fmaxf(m, L[e]);
  float z = 0.f;
  for (int e = 0; e < E; ++e) z += expf(L[e] - m);
  mz[t] = make_float2(m, z);
}

// key[r] = bits of s(src_tok[r], expert of r) for every kept row r
__global__ void __launch_bounds__(256) cap_keys_kernel(const float* __restrict__ logits,
                                                       const float2* __restrict__ mz,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ src_tok, int E,
                                                       int rows_upper, uint32_t* __restrict__ key) {
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  for (int e = threadIdx.x; e <= E; e += 256) offs[e] = offsets[e];
  __syncthreads();
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows_upper || r >= offs[E]) return;
  int lo = 0, hi = E - 1;  // expert e with offs[e] <= r < offs[e+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int t = src_tok[r];
  const float2 s = mz[t];
  key[r] = __float_as_uint(expf(logits[size_t(t) * E + lo] - s.x) / s.y);
}

__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  // exclusive prefix over the 256 threads in thread order
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += tmp[w];
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return before + x - v;
}

// One workgroup per group of experts: rows [offsets[g0], offsets[g0 + group]).
__global__ void __launch_bounds__(256) cap_select_kernel(const uint32_t* __restrict__ key,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ src_tok,
                                                         const int32_t* __restrict__ dst_row,
                                                         int k, int group, int capacity,
                                                         int32_t* __restrict__ out) {
  __shared__ int hist[256];
  __shared__ int tmp[4];
  __shared__ int sel[2];
  const int tid = threadIdx.x;
  const int g0 = blockIdx.x * group;
  const int R0 = offsets[g0], R1 = offsets[g0 + group];
  const int n = R1 - R0;
  if (n <= capacity) return;  // everything fits: nothing dropped
  // radix select of the capacity-th largest key, 8 bits at a time from the top
  uint32_t prefix = 0, pmask = 0;
  int remaining = capacity;  // keys still to take at or below the current prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += 256) hist[b] = 0;
    __syncthreads();
    for (int r = R0 + tid; r < R1; r += 256) {
      const uint32_t v = key[r];
      if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, b = 255;
      for (; b > 0; --b) {
        if (acc + hist[b] >= remaining) break;
        acc += hist[b];
      }
      sel[0] = b;
      sel[1] = remaining - acc;
    }
    __syncthreads();
    prefix |= uint32_t(sel[0]) << shift;
    pmask |= 255u << shift;
    remaining = sel[1];
    __syncthreads();
  }
  // keep keys > prefix, and the first `remaining` rows (in row order) equal to it
  int run = 0;
  for (int base = R0; base < R1; base += 256) {
    const int r = base + tid;
    const uint32_t v = r < R1 ? key[r] : 0u;
    const int tie = (r < R1 && v == prefix) ? 1 : 0;
    int total;
    const int rank = run + block_excl_scan(tie, tmp, &total);
    run += total;
    if (r < R1 && !(v > prefix || (tie && rank < remaining))) {
      const int t = src_tok[r];
      for (int j = 0; j < k; ++j)
        if (dst_row[size_t(t) * k + j] == r) out[size_t(t) * k + j] = -1;
    }
  }
}

__global__ void copy_i32_kernel(const int32_t* __restrict__ a, int n, int32_t* __restrict__ b) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) b[i] = a[i];
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

size_t capacity_ws_bytes(int T, int E, int k) {
  const size_t n = size_t(T) * k;
  return al256(size_t(E) * 4) + al256(size_t(E + 1) * 4) + 3 * al256(n * 4) + al256(size_t(T) * 8) +
         index_ws_bytes(T, E);
}

int capacity_drop(const int32_t* topk_idx, const float* logits, int T, int E, int k, int group,
                  int capacity, int32_t* out, void* ws, hipStream_t s) {
  const size_t n = size_t(T) * k;
  unsigned char* w = static_cast<unsigned char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(w);
  w += al256(size_t(E) * 4);
  int32_t* offsets = reinterpret_cast<int32_t*>(w);
  w += al256(size_t(E + 1) * 4);
  int32_t* dst_row = reinterpret_cast<int32_t*>(w);
  w += al256(n * 4);
  int32_t* src_tok = reinterpret_cast<int32_t*>(w);
  w += al256(n * 4);
  uint32_t* key = reinterpret_cast<uint32_t*>(w);
  w += al256(n * 4);
  float2* mz = reinterpret_cast<float2*>(w);
  w += al256(size_t(T) * 8);
  int rc = index_build(topk_idx, T, E, k, counts, offsets, dst_row, src_tok, w, s);
  if (rc) return rc;
  timer_begin(kTCapacity, s);
  if (out != topk_idx)
    hipLaunchKernelGGL(copy_i32_kernel, dim3(ceil_div(int(n), 256)), dim3(256), 0, s, topk_idx, int(n),
                       out);
  hipLaunchKernelGGL(cap_stats_kernel, dim3(ceil_div(T, 256)), dim3(256), 0, s, logits, T, E, mz);
  hipLaunchKernelGGL(cap_keys_kernel, dim3(ceil_div(int(n), 256)), dim3(256), 0, s, logits, mz, offsets,
                     src_tok, E, int(n), key);
  hipLaunchKernelGGL(cap_select_kernel, dim3(E / group), dim3(256), 0, s, key, offsets, src_tok,
                     dst_row, k, group, capacity, out);
  timer_end(kTCapacity, s);
  return launch_status();
}

}  // namespace moe_launch
