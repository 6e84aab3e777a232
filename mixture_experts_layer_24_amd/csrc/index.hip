// Index builder for the dispatch into expert-contiguous rows.
//
// MegaScale-MoE paper review, §四 (adaptive EP communication: an extra local
// scatter keeps each expert's tokens contiguous); research digest §3.3
// Diagram C (rows ordered by expert, then by source).  On one GPU the source
// is the token index, so row order inside an expert is ascending token.
//
// Three small kernels, all on device data (no host round trip):
//   count  -- per block of 256 tokens, a per-expert histogram in LDS;
//   scan   -- one workgroup: per-expert totals, the exclusive offsets, and each
//             block's starting row inside every expert;
//   assign -- per block again: a token's rank among the block's tokens of the
//             same expert comes from 64-bit lane masks (one per expert and
//             wave) built with LDS atomic OR, then popcount of the lanes below.
// The result is deterministic and stable whatever the scheduling.
#include "common.h"

namespace moe {

constexpr int kIdxBlock = 256;  // tokens per block in count / assign

__global__ void __launch_bounds__(kIdxBlock) idx_count_kernel(const int32_t* __restrict__ idx,
                                                              int T, int E, int k,
                                                              int32_t* __restrict__ blk_cnt) {
  __shared__ int hist[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kIdxBlock) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kIdxBlock + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      int e = idx[size_t(t) * k + j];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kIdxBlock) blk_cnt[size_t(blockIdx.x) * E + e] = hist[e];
}

// One workgroup of 256 threads.  blk_cnt [nb][E] is rewritten in place into
// each block's first row per expert.
__global__ void __launch_bounds__(256) idx_scan_kernel(int32_t* __restrict__ blk_cnt, int nb,
                                                       int E, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets) {
  __shared__ int tot[MOE_MAX_EXPERTS + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) {
    int s = 0;
    for (int b = 0; b < nb; ++b) {
      int c = blk_cnt[size_t(b) * E + e];
      blk_cnt[size_t(b) * E + e] = s;  // prefix within the expert, offset added below
      s += c;
    }
    tot[e] = s;
    counts[e] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) { int c = tot[e]; tot[e] = run; run += c; }
    tot[E] = run;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 256) offsets[e] = tot[e];
  for (int e = tid; e < E; e += 256) {
    int base = tot[e];
    for (int b = 0; b < nb; ++b) blk_cnt[size_t(b) * E + e] += base;
  }
}

__global__ void __launch_bounds__(kIdxBlock) idx_assign_kernel(const int32_t* __restrict__ idx,
                                                               int T, int E, int k,
                                                               const int32_t* __restrict__ blk_base,
                                                               int32_t* __restrict__ dst_row,
                                                               int32_t* __restrict__ src_tok) {
  constexpr int W = kIdxBlock / kWave;
  __shared__ unsigned long long mask[W][MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  for (int q = tid; q < W * E; q += kIdxBlock) mask[q / E][q % E] = 0ull;
  __syncthreads();
  const int t = blockIdx.x * kIdxBlock + tid;
  int ex[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    int e = t < T ? idx[size_t(t) * k + j] : -1;
    ex[j] = (e >= 0 && e < E) ? e : -1;
    if (ex[j] >= 0) atomicOr(&mask[wave][ex[j]], 1ull << lane);
  }
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t* base = blk_base + size_t(blockIdx.x) * E;
    for (int j = 0; j < k; ++j) {
      int e = ex[j];
      int r = -1;
      if (e >= 0) {
        r = base[e] + __popcll(mask[wave][e] & below);
        for (int w2 = 0; w2 < wave; ++w2) r += __popcll(mask[w2][e]);
        src_tok[r] = t;
      }
      dst_row[size_t(t) * k + j] = r;
    }
  }
}

// One GPU's share of the experts: ids in [e_lo, e_lo + e_count) renumbered
// from 0, every other id -1 (dropped by the index builder).
__global__ void __launch_bounds__(256) idx_local_kernel(const int32_t* __restrict__ idx, int n,
                                                        int e_lo, int e_count,
                                                        int32_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const int e = idx[i];
    out[i] = (e >= e_lo && e < e_lo + e_count) ? e - e_lo : -1;
  }
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

int local_ids(const int32_t* topk_idx, int n, int e_lo, int e_count, int32_t* out, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(idx_local_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, s, topk_idx, n, e_lo,
                       e_count, out);
  return launch_status();
}

size_t index_ws_bytes(int T, int E) {
  size_t nb = size_t(ceil_div(T > 0 ? T : 1, kIdxBlock));
  return ((nb * size_t(E) * 4 + 255) / 256) * 256;
}

int index_build(const int32_t* topk_idx, int T, int E, int k, int32_t* counts, int32_t* offsets,
                int32_t* dst_row, int32_t* src_tok, void* ws, hipStream_t s) {
  int nb = ceil_div(T, kIdxBlock);
  int32_t* blk = static_cast<int32_t*>(ws);
  timer_begin(kTIndex, s);
  if (T > 0)
    hipLaunchKernelGGL(idx_count_kernel, dim3(nb), dim3(kIdxBlock), 0, s, topk_idx, T, E, k, blk);
  hipLaunchKernelGGL(idx_scan_kernel, dim3(1), dim3(256), 0, s, blk, nb, E, counts, offsets);
  if (T > 0)
    hipLaunchKernelGGL(idx_assign_kernel, dim3(nb), dim3(kIdxBlock), 0, s, topk_idx, T, E, k, blk,
                       dst_row, src_tok);
  timer_end(kTIndex, s);
  return launch_status();
}

}  // namespace moe_launch
