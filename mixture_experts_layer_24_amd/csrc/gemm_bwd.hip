// Backward of the SwiGLU expert GroupedGEMM, routing held fixed.
//
// FC2's backward needs FC2's input and the gradient of its output, and that
// input is recomputed instead of kept (MegaScale-MoE paper review, §四
// selective activation recomputation; research digest §3.3: activation
// memory falls from a 3kf to a 2kf term).  Here the forward keeps FC1's
// output G|U (the 2kf term); A = SiLU(G)*U is recomputed in the dA epilogue.
// Weight gradients accumulate and are written in FP32 (review §三 parameter
// update: FP32 gradient accumulation).
//
// Every product runs on the same NT engine (both operands K-contiguous):
//   dA   = dYp W2^T            SchedM, B = W2 as [hf][h]  -> dG, dU, A (epilogue)
//   dXp  = [dG|dU] W13^T       SchedM, B = W13 as [h][2hf packed]
//   dW2  = A^T dYp             SchedK over transposed, zero-padded copies
//   dW13 = Xp^T [dG|dU]        SchedK, epilogue splits dW1 / dW3
// The weight-gradient products contract over each expert's rows, so their
// operands are first transposed per expert into [C][K_e] blocks with K_e the
// row count rounded up to 64 (zeros beyond it).
#include "gemm_engine.h"

namespace moe {

// Per-expert transpose with zero padding: src [rows][C] (expert-contiguous
// rows) -> dst, expert e at element kpre[e]*C laid out [C][Kp_e] with
// Kp_e = roundup(M_e, pad) (pad a multiple of 64: one 128-byte K slab of the
// GEMM's element type).  One 64 x 64 tile per workgroup through LDS.
__global__ void __launch_bounds__(256) xpose_kernel(const uint16_t* __restrict__ src, int C,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    int rows, int pad, uint16_t* __restrict__ dst) {
  __shared__ int kpre[MOE_MAX_EXPERTS + 1];
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ uint16_t tile[64][64 + 8];
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += 256) {
    int o = offsets[e];
    offs[e] = o < 0 ? 0 : (o > rows ? rows : o);
  }
  __syncthreads();
  if (tid == 0) {
    int kp = 0, prev = offs[0];
    for (int e = 0; e < E; ++e) {
      int lo = prev, hi = offs[e + 1] < prev ? prev : offs[e + 1];
      prev = hi;
      offs[e] = lo;
      kpre[e] = kp;
      kp += ((hi - lo + pad - 1) / pad) * pad;
    }
    offs[E] = prev;
    kpre[E] = kp;
  }
  __syncthreads();
  const int k0g = blockIdx.y * 64;
  if (k0g >= kpre[E]) return;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kpre[mid] <= k0g) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int k0 = k0g - kpre[e], kp = kpre[e + 1] - kpre[e], m = offs[e + 1] - offs[e];
  const int c0 = blockIdx.x * 64;
  {  // load 64 rows x 64 columns (two 16-byte chunks per thread)
    const int i = tid >> 2, cc = (tid & 3) * 16;
    u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (k0 + i < m) {
      const u32x4* p = reinterpret_cast<const u32x4*>(src + size_t(offs[e] + k0 + i) * C + c0 + cc);
      v0 = p[0];
      v1 = p[1];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[i][cc + 2 * q] = uint16_t(v0[q]);
      tile[i][cc + 2 * q + 1] = uint16_t(v0[q] >> 16);
      tile[i][cc + 8 + 2 * q] = uint16_t(v1[q]);
      tile[i][cc + 8 + 2 * q + 1] = uint16_t(v1[q] >> 16);
    }
  }
  __syncthreads();
  {  // write 64 output rows (columns of src) x 64 k values
    const int c = tid >> 2, kk = (tid & 3) * 16;
    u32x4 w0, w1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w0[q] = uint32_t(tile[kk + 2 * q][c]) | (uint32_t(tile[kk + 2 * q + 1][c]) << 16);
      w1[q] = uint32_t(tile[kk + 8 + 2 * q][c]) | (uint32_t(tile[kk + 8 + 2 * q + 1][c]) << 16);
    }
    u32x4* d = reinterpret_cast<u32x4*>(dst + size_t(kpre[e]) * C + size_t(c0 + c) * kp + k0 + kk);
    d[0] = w0;
    d[1] = w1;
  }
}

// Rows r < n of length len (a multiple of 8): codes and scale[r].
__global__ void __launch_bounds__(256) rowq_kernel(const uint16_t* __restrict__ src, int n, int len,
                                                   uint8_t* __restrict__ dst,
                                                   float* __restrict__ scale) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  rowq_wave(src + size_t(r) * len, len, dst + size_t(r) * len, scale + r);
}

// The per-expert transposed blocks of xpose_kernel, quantized row by row:
// row c of expert e (length Kp_e, at kpre[e]*C + c*Kp_e) -> codes at the same
// place, scale[e][c] (1 for an expert without rows).  The zero padding
// changes neither the scale nor the sums.
__global__ void __launch_bounds__(256) rowq_xposed_kernel(const uint16_t* __restrict__ src, int C,
                                                          const int32_t* __restrict__ offsets,
                                                          int E, int rows, int pad,
                                                          uint8_t* __restrict__ dst,
                                                          float* __restrict__ scale) {
  __shared__ int kpre[MOE_MAX_EXPERTS + 1];
  if (threadIdx.x == 0) {
    int kp = 0, prev = 0;
    for (int e = 0; e < E; ++e) {
      int o0 = offsets[e], o1 = offsets[e + 1];
      o0 = o0 < 0 ? 0 : (o0 > rows ? rows : o0);
      o1 = o1 < 0 ? 0 : (o1 > rows ? rows : o1);
      const int lo = e == 0 ? o0 : prev, hi = o1 < lo ? lo : o1;
      prev = hi;
      kpre[e] = kp;
      kp += ((hi - lo + pad - 1) / pad) * pad;
    }
    kpre[E] = kp;
  }
  __syncthreads();
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);  // r = e * C + c
  if (r >= E * C) return;
  const int e = r / C, c = r - e * C;
  const int kp = kpre[e + 1] - kpre[e];
  if (kp == 0) {
    if ((threadIdx.x & 63) == 0) scale[r] = 1.0f;
    return;
  }
  const size_t base = size_t(kpre[e]) * C + size_t(c) * kp;
  rowq_wave(src + base, kp, dst + base, scale + r);
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

using CfgB = CfgFor<MOE_BF16>::type;
// dA stages the kept G|U through the one LDS stage idle during its epilogue:
// 128-byte slabs in two stages leave 8 KB per wave there (64 rows at a time).
using CfgDA = GemmCfg<2, 4, 4, 2, 1, 128, 2>;

static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// Upper bound of the padded K extent: sum_e roundup(M_e, pad) <= rows + (pad-1) E.
static size_t kpad_upper(int rows, int E, int pad = kpad_elems<MOE_BF16>()) {
  return size_t(rows) + size_t(pad - 1) * E;
}

size_t grouped_bwd_ws_bytes(int rows, int h, int h_ffn, int E, int dtype) {
  (void)dtype;
  const size_t r = size_t(rows), hh = size_t(h), hf = size_t(h_ffn), kp = kpad_upper(rows, E);
  return al256(r * 2 * hf * 2)          // dG|dU, packed like G|U
         + al256(r * hf * 2)            // A recomputed
         + 2 * al256(hh * kp * 2)       // Xp^T, dYp^T
         + al256(hf * kp * 2)           // A^T
         + al256(2 * hf * kp * 2)       // (dG|dU)^T
         + splitk_ws_bytes<CfgB>();   // split-K partial tiles
}

static int xpose(const void* src, int C, const int32_t* offsets, int E, int rows, void* dst,
                 hipStream_t s, int pad = kpad_elems<MOE_BF16>()) {
  const size_t ky = (kpad_upper(rows, E, pad) + 63) / 64;
  hipLaunchKernelGGL(xpose_kernel, dim3(C / 64, unsigned(ky)), dim3(256), 0, s,
                     (const uint16_t*)src, C, offsets, E, rows, pad, (uint16_t*)dst);
  return launch_status();
}

int grouped_bwd(const void* dyp, const void* xp, const void* h13_save, const moe_weights* W,
                const int32_t* offsets, int rows, void* dxp, float* dw1, float* dw3, float* dw2,
                void* ws, hipStream_t s) {
  const int h = W->h, hf = W->h_ffn, E = W->E;
  unsigned char* w = static_cast<unsigned char*>(ws);
  const size_t r = size_t(rows), kp = kpad_upper(rows, E);
  void* dgu = w;
  w += al256(r * 2 * hf * 2);
  void* act = w;
  w += al256(r * hf * 2);
  void* xpT = w;
  w += al256(size_t(h) * kp * 2);
  void* dypT = w;
  w += al256(size_t(h) * kp * 2);
  void* actT = w;
  w += al256(size_t(hf) * kp * 2);
  void* dguT = w;
  w += al256(2 * size_t(hf) * kp * 2);
  void* split_ws = w;
  int rc;

  timer_begin(kTXpose, s);
  if ((rc = xpose(xp, h, offsets, E, rows, xpT, s))) return rc;
  if ((rc = xpose(dyp, h, offsets, E, rows, dypT, s))) return rc;
  timer_end(kTXpose, s);

  // dA = dYp W2^T, with dG, dU and A formed in the epilogue
  GemmArgs ga{dyp, nullptr, W->w2_bwd, nullptr, offsets, E, h, hf, rows, 0,
              dgu, act, const_cast<void*>(h13_save), nullptr, nullptr, nullptr};
  splitk_ws_set<CfgDA>(ga, split_ws);
  if ((rc = launch_gemm<CfgDA, MOE_BF16, kModeBwdDA, kSchedM>(ga, kTBwd1, s)))
    return rc;

  timer_begin(kTXpose, s);
  if ((rc = xpose(act, hf, offsets, E, rows, actT, s))) return rc;
  if ((rc = xpose(dgu, 2 * hf, offsets, E, rows, dguT, s))) return rc;
  timer_end(kTXpose, s);

  // dW2 = A^T dYp  (per expert [hf][h], fp32)
  GemmArgs g2{actT, nullptr, dypT, nullptr, offsets, E, 0, h, rows, hf,
              dw2, nullptr, nullptr, nullptr, nullptr, nullptr};
  splitk_ws_set<CfgB>(g2, split_ws);
  if ((rc = launch_gemm<CfgB, MOE_BF16, kModeDW, kSchedK>(g2, kTBwd2, s)))
    return rc;

  // dXp = [dG|dU] W13^T
  GemmArgs g3{dgu, nullptr, W->w13_bwd, nullptr, offsets, E, 2 * hf, h, rows, 0,
              dxp, nullptr, nullptr, nullptr, nullptr, nullptr};
  splitk_ws_set<CfgB>(g3, split_ws);
  if ((rc = launch_gemm<CfgB, MOE_BF16, kModeFC2, kSchedM>(g3, kTBwd3, s)))
    return rc;

  // dW1 | dW3 = Xp^T [dG|dU]  (per expert [h][hf] each, fp32)
  GemmArgs g4{xpT, nullptr, dguT, nullptr, offsets, E, 0, 2 * hf, rows, h,
              dw1, dw3, nullptr, nullptr, nullptr, nullptr};
  splitk_ws_set<CfgB>(g4, split_ws);
  return launch_gemm<CfgB, MOE_BF16, kModeDW13, kSchedK>(g4, kTBwd4, s);
}

}  // namespace moe_launch

namespace moe_launch {
using namespace moe;

using CfgQ = CfgFor<MOE_FP8_E4M3>::type;
static_assert(CfgQ::kRowB == CfgDA::kRowB && CfgQ::kStages == CfgDA::kStages &&
                  CfgQ::kBM == CfgDA::kBM && CfgQ::kBN == CfgDA::kBN,
              "the FP8 dA epilogue stages G|U like the BF16 one");

// FP8 backward workspace: bf16 dG|dU and A, dG|dU codes + row scales, one
// bf16 transposed block reused for each operand, the four transposed code
// blocks and their per-expert channel scales, split-K partials.
size_t grouped_bwd_fp8_ws_bytes(int rows, int h, int h_ffn, int E) {
  const size_t r = size_t(rows), hh = size_t(h), hf = size_t(h_ffn), e = size_t(E);
  const size_t kp = kpad_upper(rows, E, kpad_elems<MOE_FP8_E4M3>());
  const size_t cmax = hh > 2 * hf ? hh : 2 * hf;
  return al256(r * 2 * hf * 2) + al256(r * hf * 2) + al256(r * 2 * hf) + al256(r * 4) +
         al256(cmax * kp * 2) + 2 * al256(hh * kp) + al256(hf * kp) + al256(2 * hf * kp) +
         2 * al256(e * hh * 4) + al256(e * hf * 4) + al256(e * 2 * hf * 4) + splitk_ws_bytes<CfgQ>();
}

static int xpose_q(const void* src, int C, const int32_t* offsets, int E, int rows, void* tmp,
                   void* dst, float* scale, hipStream_t s) {
  constexpr int pad = kpad_elems<MOE_FP8_E4M3>();
  int rc = xpose(src, C, offsets, E, rows, tmp, s, pad);
  if (rc) return rc;
  hipLaunchKernelGGL(rowq_xposed_kernel, dim3(ceil_div(E * C, 4)), dim3(256), 0, s,
                     (const uint16_t*)tmp, C, offsets, E, rows, pad, (uint8_t*)dst, scale);
  return launch_status();
}

int grouped_bwd_fp8(const void* dyp_q, const float* dyp_scale, const void* dyp, const void* xp,
                    const void* h13_save, const moe_weights* W, const int32_t* offsets, int rows,
                    void* dxp, float* dw1, float* dw3, float* dw2, void* ws, hipStream_t s) {
  const int h = W->h, hf = W->h_ffn, E = W->E;
  const size_t r = size_t(rows), kp = kpad_upper(rows, E, kpad_elems<MOE_FP8_E4M3>());
  const size_t cmax = size_t(h) > 2 * size_t(hf) ? size_t(h) : 2 * size_t(hf);
  unsigned char* w = static_cast<unsigned char*>(ws);
  auto take = [&](size_t bytes) { unsigned char* p = w; w += al256(bytes); return p; };
  void* dgu = take(r * 2 * hf * 2);
  void* act = take(r * hf * 2);
  void* dgu_q = take(r * 2 * hf);
  float* dgu_s = reinterpret_cast<float*>(take(r * 4));
  void* tmp = take(cmax * kp * 2);
  void* xpT = take(size_t(h) * kp);
  void* dypT = take(size_t(h) * kp);
  void* actT = take(size_t(hf) * kp);
  void* dguT = take(2 * size_t(hf) * kp);
  float* sx = reinterpret_cast<float*>(take(size_t(E) * h * 4));
  float* sd = reinterpret_cast<float*>(take(size_t(E) * h * 4));
  float* sa = reinterpret_cast<float*>(take(size_t(E) * hf * 4));
  float* sg = reinterpret_cast<float*>(take(size_t(E) * 2 * hf * 4));
  void* split_ws = w;
  int rc;

  timer_begin(kTXpose, s);
  if ((rc = xpose_q(xp, h, offsets, E, rows, tmp, xpT, sx, s))) return rc;
  if ((rc = xpose_q(dyp, h, offsets, E, rows, tmp, dypT, sd, s))) return rc;
  timer_end(kTXpose, s);

  // dA = dYp W2^T on FP8 codes; epilogue rescales and forms dG, dU and A
  GemmArgs ga{dyp_q, dyp_scale, W->w2_bwd, W->w2_bwd_scale, offsets, E, h, hf, rows, 0,
              dgu, act, const_cast<void*>(h13_save), nullptr, nullptr, nullptr};
  splitk_ws_set<CfgQ>(ga, split_ws);
  if ((rc = launch_gemm<CfgQ, MOE_FP8_E4M3, kModeBwdDA, kSchedM>(ga, kTBwd1, s))) return rc;

  timer_begin(kTQuant, s);
  hipLaunchKernelGGL(rowq_kernel, dim3(ceil_div(rows, 4)), dim3(256), 0, s, (const uint16_t*)dgu, rows,
                     2 * hf, (uint8_t*)dgu_q, dgu_s);
  timer_end(kTQuant, s);
  timer_begin(kTXpose, s);
  if ((rc = xpose_q(act, hf, offsets, E, rows, tmp, actT, sa, s))) return rc;
  if ((rc = xpose_q(dgu, 2 * hf, offsets, E, rows, tmp, dguT, sg, s))) return rc;
  timer_end(kTXpose, s);

  // dW2 = A^T dYp  (per expert [hf][h], fp32)
  GemmArgs g2{actT, sa, dypT, sd, offsets, E, 0, h, rows, hf, dw2, nullptr, nullptr, nullptr,
              nullptr, nullptr};
  splitk_ws_set<CfgQ>(g2, split_ws);
  if ((rc = launch_gemm<CfgQ, MOE_FP8_E4M3, kModeDW, kSchedK>(g2, kTBwd2, s))) return rc;

  // dXp = [dG|dU] W13^T
  GemmArgs g3{dgu_q, dgu_s, W->w13_bwd, W->w13_bwd_scale, offsets, E, 2 * hf, h, rows, 0, dxp,
              nullptr, nullptr, nullptr, nullptr, nullptr};
  splitk_ws_set<CfgQ>(g3, split_ws);
  if ((rc = launch_gemm<CfgQ, MOE_FP8_E4M3, kModeFC2, kSchedM>(g3, kTBwd3, s))) return rc;

  // dW1 | dW3 = Xp^T [dG|dU]
  GemmArgs g4{xpT, sx, dguT, sg, offsets, E, 0, 2 * hf, rows, h, dw1, dw3, nullptr, nullptr,
              nullptr, nullptr};
  splitk_ws_set<CfgQ>(g4, split_ws);
  return launch_gemm<CfgQ, MOE_FP8_E4M3, kModeDW13, kSchedK>(g4, kTBwd4, s);
}

}  // namespace moe_launch
