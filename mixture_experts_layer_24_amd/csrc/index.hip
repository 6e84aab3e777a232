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
//             block's starting row inside every expert (threads split the
//             blocks of an expert into ranges);
//   assign -- per block again: a token's rank among the block's tokens of the
//             same expert comes from 64-bit lane masks (one per expert and
//             wave) built with LDS atomic OR, then popcount of the lanes below;
//             a block where some token names an expert twice counts pairs per
//             slot position instead, so those pairs take consecutive rows.
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
// each block's first row per expert.  G = 256 / E threads (rounded down to a
// power of two) share an expert, thread g owning a contiguous range of
// blocks: it sums its range, the range sums are scanned per expert, the
// expert totals across experts, and each thread then writes its range's
// running offsets.  Loads go in batches of eight, so the chain of dependent
// global reads is ~nb / (8 G) long instead of nb.
__global__ void __launch_bounds__(256) idx_scan_kernel(int32_t* __restrict__ blk_cnt, int nb,
                                                       int E, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets) {
  __shared__ int tot[MOE_MAX_EXPERTS + 1];
  __shared__ int part[256];
  const int tid = threadIdx.x;
  int G = 1;
  while (G * 2 * E <= 256) G *= 2;
  const int e = tid / G, g = tid - e * G;
  const bool act = e < E;
  const int b0 = act ? int(int64_t(nb) * g / G) : 0;
  const int b1 = act ? int(int64_t(nb) * (g + 1) / G) : 0;
  int s = 0;
  for (int b = b0; b < b1; b += 8) {
    int c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = b + i < b1 ? blk_cnt[size_t(b + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += c[i];
  }
  part[tid] = s;
  __syncthreads();
  if (tid < E) {  // exclusive scan of expert tid's range sums
    int run = 0;
    for (int q = 0; q < G; ++q) {
      const int v = part[tid * G + q];
      part[tid * G + q] = run;
      run += v;
    }
    tot[tid] = run;
    counts[tid] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int x = 0; x < E; ++x) { const int c = tot[x]; tot[x] = run; run += c; }
    tot[E] = run;
  }
  __syncthreads();
  for (int x = tid; x <= E; x += 256) offsets[x] = tot[x];
  if (act) {
    int r = tot[e] + part[tid];
    for (int b = b0; b < b1; b += 8) {
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = b + i < b1 ? blk_cnt[size_t(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (b + i < b1) blk_cnt[size_t(b + i) * E + e] = r;
        r += c[i];
      }
    }
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
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int ex[MOE_MAX_TOPK];
  int dup = 0;  // this token names one expert in two of its slots
  for (int j = 0; j < k; ++j) {
    int e = t < T ? idx[size_t(t) * k + j] : -1;
    ex[j] = (e >= 0 && e < E) ? e : -1;
    for (int j2 = 0; j2 < j; ++j2) dup |= ex[j] >= 0 && ex[j2] == ex[j];
    if (ex[j] >= 0) atomicOr(&mask[wave][ex[j]], 1ull << lane);
  }
  if (!__syncthreads_or(dup)) {
    // every token counts at most once per expert: its rank among the
    // block's pairs of that expert is the number of lanes below it (this
    // wave) and in earlier waves that name the expert
    if (t < T) {
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
    return;
  }
  // A token of this block names some expert twice: its pairs of that expert
  // take consecutive rows in slot order (the order of (token, slot) pairs).
  // Count, per slot position jj in turn, the pairs of earlier tokens at that
  // position (masks rebuilt per position), plus the token's own earlier
  // slots with the same expert.
  int acc[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    acc[j] = 0;
    for (int j2 = 0; j2 < j; ++j2) acc[j] += ex[j] >= 0 && ex[j2] == ex[j];
  }
  for (int jj = 0; jj < k; ++jj) {
    __syncthreads();  // the previous position's masks are read out
    for (int q = tid; q < W * E; q += kIdxBlock) mask[q / E][q % E] = 0ull;
    __syncthreads();
    if (ex[jj] >= 0) atomicOr(&mask[wave][ex[jj]], 1ull << lane);
    __syncthreads();
    for (int j = 0; j < k; ++j) {
      const int e = ex[j];
      if (e < 0) continue;
      acc[j] += __popcll(mask[wave][e] & below);
      for (int w2 = 0; w2 < wave; ++w2) acc[j] += __popcll(mask[w2][e]);
    }
  }
  if (t < T) {
    const int32_t* base = blk_base + size_t(blockIdx.x) * E;
    for (int j = 0; j < k; ++j) {
      const int r = ex[j] >= 0 ? base[ex[j]] + acc[j] : -1;
      if (r >= 0) src_tok[r] = t;
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
