// Dispatch copy and FC1 overlapped by tile arrival, on one GPU.
//
// The pages overlap the expert GroupedGEMM with the communication that feeds
// it: tiles of the dispatched rows arrive over time, each is flagged on the
// device as it lands, and the GEMM starts a tile once its rows are flagged,
// instead of waiting for the whole exchange (MegaScale-MoE research digest
// §3.3 Diagram C; paper review §四 intra-operator overlap).  On one GPU the
// dispatch copy into expert-contiguous rows stands in for the exchange: it
// runs as a producer kernel on a second stream, writes the routed rows in row
// order, and counts each expert's rows as they land; FC1 (GemmArgs::ready,
// mode kModeFC1Arr) waits until all of a tile's expert has landed before
// loading the tile's first slab.  The flag is per expert, not per 256-row
// tile: E + 1 counters, and the workgroups of one XCD, which take the row
// tiles of an expert against a few weight blocks, start together; flags per
// row tile measured the same.  FC2 then runs as in the plain forward.
// The copy, FC1 and FC2 compute exactly what moe_permute and
// moe_grouped_swiglu_fwd compute, so the results are the same bit for bit.
//
// Forward progress: FC1 takes one workgroup per CU (130 KB of LDS, two waves
// of ~200 VGPRs per SIMD); a copy workgroup (four waves of few VGPRs, 1 KB of
// LDS) fits beside it on every CU, so the copy always finds room while FC1
// waits, and FC1's waits are bounded (status 1 if one gives up).
#include <mutex>

#include "gemm_engine.h"

namespace moe {

constexpr int kArrRows = 32;  // routed rows per copy workgroup
constexpr int kArrU = 8;      // 16-byte loads in flight per thread

// Xp[r] = x[src_tok[r]] for the kept rows r < offsets[E], kArrRows rows per
// workgroup in row order; then a device-scope release and, per expert the
// workgroup's rows belong to, an add of its row count to ready[e]; then an add
// of all its rows to `done`.
__global__ void __launch_bounds__(256) dispatch_flag_kernel(const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ src_tok,
                                                            const int32_t* __restrict__ offsets, int E,
                                                            int h, uint16_t* __restrict__ xp,
                                                            uint32_t* __restrict__ ready,
                                                            uint32_t* __restrict__ done) {
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  const int tid = threadIdx.x;
  if (tid == 0) {  // offsets clamped and non-decreasing, as the GEMM reads them
    int prev = 0;
    for (int e = 0; e <= E; ++e) {
      int o = offsets[e];
      o = o < prev ? prev : o;
      offs[e] = o;
      prev = o;
    }
  }
  __syncthreads();
  const int rows = offs[E], r0 = blockIdx.x * kArrRows;
  if (r0 >= rows) return;  // uniform in the workgroup
  const int r1 = r0 + kArrRows < rows ? r0 + kArrRows : rows;
  // Beside the GEMM this kernel gets a few waves per CU, so each thread keeps
  // kArrU 16-byte loads in flight (the rows' tokens are read once, into LDS).
  __shared__ int tok[kArrRows];
  if (tid < r1 - r0) tok[tid] = src_tok[r0 + tid];
  __syncthreads();
  const int nch = h / 8;  // 16-byte chunks per row
  const int n = (r1 - r0) * nch;
  for (int i0 = tid; i0 < n; i0 += kArrU * 256) {
    u32x4 v[kArrU];
#pragma unroll
    for (int u = 0; u < kArrU; ++u) {
      const int i = i0 + u * 256, rr = i / nch, c = i - rr * nch;
      if (i < n) v[u] = reinterpret_cast<const u32x4*>(x + size_t(tok[rr]) * h)[c];
    }
#pragma unroll
    for (int u = 0; u < kArrU; ++u) {
      const int i = i0 + u * 256, rr = i / nch, c = i - rr * nch;
      if (i < n) reinterpret_cast<u32x4*>(xp + size_t(r0 + rr) * h)[c] = v[u];
    }
  }
  // release only (agent scope): this thread's rows before the counts
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    for (int r = r0; r < r1;) {
      int lo = 0, hi = E - 1;  // the expert e with offs[e] <= r < offs[e + 1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= r) lo = mid; else hi = mid - 1;
      }
      const int n = (r1 < offs[lo + 1] ? r1 : offs[lo + 1]) - r;
      atomicAdd(ready + lo, uint32_t(n));
      r += n;
    }
    atomicAdd(done, uint32_t(r1 - r0));
  }
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

using CfgA = CfgFor<MOE_BF16>::type;

static size_t al256a(size_t x) { return (x + 255) & ~size_t(255); }

size_t arrival_ws_bytes(int T, int k, int h, int h_ffn, int E) {
  const int rows = T * k;
  return al256a(index_ws_bytes(T, E)) + al256a((size_t(E) + 1) * 4) +
         grouped_fwd_ws_bytes(rows > 0 ? rows : 1, h, h_ffn, E, MOE_BF16);
}

namespace {
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];  // per device
}  // namespace

// The copy's stream (non-blocking, so it never waits for the null stream) and
// the two events that order it after the caller's earlier work and the
// caller's later work after it; created once per device.
static int side_stream(SideStream** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_side_mu);
  SideStream& ss = g_side[dev];
  if (ss.s == nullptr) {
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) return MOE_ERR_HIP;
    if (hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      return MOE_ERR_HIP;
  }
  *out = &ss;
  return MOE_OK;
}

int dispatch_swiglu_fwd(const void* x, const int32_t* topk_idx, int T, int k, int32_t* counts,
                        int32_t* offsets, int32_t* dst_row, int32_t* src_tok, const moe_weights* W,
                        void* xp, void* h13_save, void* yp, int yp_f32, int32_t* status, void* ws,
                        hipStream_t s, int spin_limit, bool copy) {
  const int h = W->h, hf = W->h_ffn, E = W->E, rows = T * k;
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* iws = w;
  w += al256a(index_ws_bytes(T, E));
  uint32_t* ready = reinterpret_cast<uint32_t*>(w);
  const int nflag = E + 1;  // rows landed per expert, then in all
  uint32_t* done = ready + (nflag - 1);
  w += al256a(size_t(nflag) * 4);
  void* act = w;
  void* split_ws = w + al256a(size_t(rows) * hf * 2);
  int rc = index_build(topk_idx, T, E, k, counts, offsets, dst_row, src_tok, iws, s);
  if (rc) return rc;
  hipLaunchKernelGGL(zero_u32_kernel<0>, dim3(ceil_div(nflag, 256)), dim3(256), 0, s, ready, nflag);
  hipLaunchKernelGGL(zero_u32_kernel<0>, dim3(1), dim3(1), 0, s, reinterpret_cast<uint32_t*>(status), 1);
  if ((rc = launch_status())) return rc;
  if (rows == 0) return MOE_OK;
  SideStream* ss = nullptr;
  if (copy && (rc = side_stream(&ss))) return rc;
  // the copy on the side stream, after everything enqueued so far (left out
  // only to test FC1's bounded waits)
  if (copy) {
    if (hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
      return MOE_ERR_HIP;
    timer_begin(kTPermute, ss->s);
    hipLaunchKernelGGL(dispatch_flag_kernel, dim3(ceil_div(rows, kArrRows)), dim3(256), 0, ss->s,
                       static_cast<const uint16_t*>(x), src_tok, offsets, E, h,
                       static_cast<uint16_t*>(xp), ready, done);
    timer_end(kTPermute, ss->s);
    if (hipEventRecord(ss->join, ss->s) != hipSuccess) return MOE_ERR_HIP;
  }
  // FC1 on the caller's stream, each row tile waiting for its rows
  GemmArgs a1{xp, nullptr, W->w13, nullptr, offsets, E, h, 2 * hf, rows, 0,
              act, nullptr, h13_save, nullptr, nullptr, nullptr, 0, ready, done, status, spin_limit};
  splitk_ws_set<CfgA>(a1, split_ws);
  if ((rc = launch_gemm<CfgA, MOE_BF16, kModeFC1Arr, kSchedM>(a1, kTFc1, s))) return rc;
  // the caller's later work (FC2 first) after the copy
  if (copy && hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return MOE_ERR_HIP;
  GemmArgs a2{act, nullptr, W->w2, nullptr, offsets, E, hf, h, rows, 0, yp, nullptr, nullptr, nullptr,
              nullptr, nullptr, yp_f32};
  splitk_ws_set<CfgA>(a2, split_ws);
  return launch_gemm<CfgA, MOE_BF16, kModeFC2, kSchedM>(a2, kTFc2, s);
}

}  // namespace moe_launch
