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
// Every product runs on the same engine:
//   dA   = dYp W2^T            SchedM, B = W2 as [hf][h]  -> dG, dU, A (epilogue)
//   dXp  = [dG|dU] W13^T       SchedM, B = W13 as [h][2hf packed]
//   dW2  = A^T dYp             SchedKR (BF16) / SchedK (FP8)
//   dW13 = Xp^T [dG|dU]        the same; the epilogue splits dW1 / dW3
// The weight-gradient products contract over each expert's rows.  In BF16
// they read the row-major routed arrays directly (the LDS transpose read
// turns the M-major slabs into MFMA fragments).  In FP8 the operands are
// quantized per channel over the expert's rows, so they are first transposed
// per expert into [C][K_e] code blocks with K_e the row count rounded up to
// 128 (zeros beyond it), the quantization done in the same pass; Xp and
// w * dY are gathered there from the token-major x and dY (no routed bf16
// copies of either), A and dG|dU read as the dA epilogue stored them.
#include "gemm_engine.h"

namespace moe {

// Per-expert quantizing transpose with zero padding: src [rows][C] bf16
// (expert-contiguous rows, C a multiple of 64) -> dst E4M3 codes, expert e at
// element kpre[e]*C laid out [C][Kp_e] with Kp_e = roundup(M_e, pad) (pad a
// multiple of 64: one 128-byte K slab of the GEMM's element type) and zeros
// beyond M_e.
//
// A work item is (64 columns, expert); workgroups take items i, i + G, ...
// (G = gridDim.x), the 64-column strips of one expert being consecutive items.
// An item walks the expert's rows in blocks of 64: each thread loads 16 bytes
// of two adjacent rows (eight threads cover a 128-byte row segment), packs the
// two rows' values of each column into one 32-bit word in LDS (column-major,
// 33 words per column: conflict-free stores), then reads 8 words = 16
// consecutive rows of one column and stores their codes contiguously.  The
// loads of the next two blocks are in flight during this block's LDS work.
//
// Codes are quantized per channel over the expert's rows (scale[e][c] =
// amax / 448, 1 for a zero channel or an expert without rows).  With
// have_amax, scale[e][c] holds the column amax on entry (the dA epilogue
// takes it for A and dG|dU); otherwise a first pass over the same rows takes
// it, and the second pass re-reads them from the Infinity Cache when the
// strips of the items in progress fit there, which the launcher arranges by
// bounding the grid.
//
// With row_src, src is token-major ([ntok][C]) and routed row r is gathered
// from token row row_src[r] - 1 (x for Xp; 0 marks a row no pair targets,
// which reads as zeros); with row_w too, each value becomes bf16(row_w[r] * v),
// the value the weighted dispatch copy stores (dY for dYp).  The routed copies
// are then never written.
__global__ void __launch_bounds__(256) xpose_kernel(const uint16_t* __restrict__ src, int C,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    int rows, int pad, void* __restrict__ dst,
                                                    float* __restrict__ scale, int have_amax,
                                                    const int32_t* __restrict__ row_src,
                                                    const float* __restrict__ row_w, int ntok) {
  __shared__ int kpre[MOE_MAX_EXPERTS + 1];
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ uint32_t tile[64 * 33];
  __shared__ float cscale[64];
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += 256) {
    const int o = offsets[e];
    offs[e] = o < 0 ? 0 : (o > rows ? rows : o);
  }
  __syncthreads();
  if (tid == 0) {
    int kp = 0, prev = offs[0];
    for (int e = 0; e < E; ++e) {
      const int lo = prev, hi = offs[e + 1] < prev ? prev : offs[e + 1];
      prev = hi;
      offs[e] = lo;
      kpre[e] = kp;
      kp += ((hi - lo + pad - 1) / pad) * pad;
    }
    offs[E] = prev;
    kpre[E] = kp;
  }
  __syncthreads();
  const int q = tid & 7, p = tid >> 3;  // 8-column chunk, row pair
  const int ns = C / 64;
  // every barrier below is reached by the whole workgroup: the item loop's
  // bounds and kp are uniform
  for (int item = blockIdx.x; item < ns * E; item += gridDim.x) {
    const int e = item / ns, c0 = (item - e * ns) * 64;
    const int r0 = offs[e], m = offs[e + 1] - r0, kp = kpre[e + 1] - kpre[e];
    if (kp == 0) {
      if (tid < 64 && c0 + tid < C) scale[size_t(e) * C + c0 + tid] = 1.0f;
      continue;
    }
    const uint16_t* sp = src + size_t(r0) * C + c0 + q * 8;
    auto ld = [&](int r) {
      u32x4 v = {0, 0, 0, 0};
      if (r < m) v = *reinterpret_cast<const u32x4*>(sp + size_t(r) * C);
      return v;
    };
    // the encoding pass is the rows' last use: nontemporal loads (DeepSeekMoE-
    // shaped FP8 step: the four transposes 1.09 -> 0.95 ms)
    auto ldn = [&](int r) {
      u32x4 v = {0, 0, 0, 0};
      if (r < m) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sp + size_t(r) * C));
      return v;
    };
    // Gathered rows: the row's token (loaded a step ahead of its data, so the
    // data load does not wait on it), the token row's chunk, and the row's
    // weight, applied where the value is used, as the weighted dispatch copy
    // rounds it.  A gathered token row serves its other routed rows too, so
    // it keeps the plain loads.
    auto gidx = [&](int r) { return r < m ? row_src[r0 + r] : 0; };
    auto graw = [&](int t1) {
      u32x4 v = {0, 0, 0, 0};
      if (t1 > 0 && t1 <= ntok) v = *reinterpret_cast<const u32x4*>(src + size_t(t1 - 1) * C + c0 + q * 8);
      return v;
    };
    auto gw = [&](int r) { return row_w && r < m ? row_w[r0 + r] : 1.0f; };
    auto weigh = [&](u32x4 v, float w) {
      if (row_w) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(bf16_lo(v[i]) * w, bf16_hi(v[i]) * w);
      }
      return v;
    };
    if (have_amax) {
      if (tid < 64 && c0 + tid < C) {
        const float a = scale[size_t(e) * C + c0 + tid];
        const float sc = a > 0.f ? a / 448.0f : 1.0f;
        cscale[tid] = sc;
        scale[size_t(e) * C + c0 + tid] = sc;
      }
      __syncthreads();
    } else {
      float am[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) am[j] = 0.f;
      // four rows per thread in flight (rows past the expert read as zeros)
      int ti[4];
      if (row_src)
#pragma unroll
        for (int u = 0; u < 4; ++u) ti[u] = gidx(p + 32 * u);
      for (int r = p; r < m; r += 128) {
        u32x4 v[4];
        if (row_src) {
          int tn[4];
          float wv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) tn[u] = gidx(r + 128 + 32 * u);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            v[u] = graw(ti[u]);
            wv[u] = gw(r + 32 * u);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            v[u] = weigh(v[u], wv[u]);
            ti[u] = tn[u];
          }
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = ld(r + 32 * u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            am[2 * i] = fmaxf(am[2 * i], fabsf(bf16_lo(v[u][i])));
            am[2 * i + 1] = fmaxf(am[2 * i + 1], fabsf(bf16_hi(v[u][i])));
          }
      }
      float* red = reinterpret_cast<float*>(tile);
#pragma unroll
      for (int j = 0; j < 8; ++j) red[(q * 8 + j) * 33 + p] = am[j];
      __syncthreads();
      if (tid < 64) {
        float a = 0.f;
        for (int i = 0; i < 32; ++i) a = fmaxf(a, red[tid * 33 + i]);
        const float sc = a > 0.f ? a / 448.0f : 1.0f;
        cscale[tid] = sc;
        if (c0 + tid < C) scale[size_t(e) * C + c0 + tid] = sc;
      }
      __syncthreads();
    }
    const int c = tid >> 2, kk = (tid & 3) * 16;  // output column, first of its 16 rows
    const size_t obase = size_t(kpre[e]) * C + size_t(c0 + c) * kp + kk;
    const float sc = cscale[c];
    const QuotScale qs = quot_scale(sc);
    // one 64-row block: the thread's rows 2p, 2p + 1 (va, vb) into the LDS
    // tile, then 16 consecutive rows of one column out, encoded
    auto encode = [&](int k0, const u32x4& va, const u32x4& vb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tile[(q * 8 + 2 * i) * 33 + p] = (va[i] & 0xFFFFu) | (vb[i] << 16);
        tile[(q * 8 + 2 * i + 1) * 33 + p] = (va[i] >> 16) | (vb[i] & 0xFFFF0000u);
      }
      __syncthreads();
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = tile[c * 33 + (kk >> 1) + i];
      if (c0 + c < C) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = e4m3x4_quot(bf16_lo(w[2 * i]), bf16_hi(w[2 * i]), bf16_lo(w[2 * i + 1]),
                             bf16_hi(w[2 * i + 1]), qs);
        *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(dst) + obase + k0) = o;
      }
      __syncthreads();
    };
    if (row_src) {
      // data two 64-row blocks ahead of the LDS work, tokens three
      int fia = gidx(128 + 2 * p), fib = gidx(129 + 2 * p);
      u32x4 va = graw(gidx(2 * p)), vb = graw(gidx(2 * p + 1));
      u32x4 na = graw(gidx(64 + 2 * p)), nb = graw(gidx(65 + 2 * p));
      float wa = gw(2 * p), wb = gw(2 * p + 1), nwa = gw(64 + 2 * p), nwb = gw(65 + 2 * p);
      for (int k0 = 0; k0 < kp; k0 += 64) {
        const int xa = gidx(k0 + 192 + 2 * p), xb = gidx(k0 + 193 + 2 * p);
        const u32x4 fa = graw(fia), fb = graw(fib);
        const float fwa = gw(k0 + 128 + 2 * p), fwb = gw(k0 + 129 + 2 * p);
        encode(k0, weigh(va, wa), weigh(vb, wb));
        va = na;
        vb = nb;
        wa = nwa;
        wb = nwb;
        na = fa;
        nb = fb;
        nwa = fwa;
        nwb = fwb;
        fia = xa;
        fib = xb;
      }
    } else {
      // loads run two 64-row blocks ahead of the LDS work
      u32x4 va = ldn(2 * p), vb = ldn(2 * p + 1), na = ldn(64 + 2 * p), nb = ldn(65 + 2 * p);
      for (int k0 = 0; k0 < kp; k0 += 64) {
        const u32x4 fa = ldn(k0 + 128 + 2 * p), fb = ldn(k0 + 129 + 2 * p);
        encode(k0, va, vb);
        va = na;
        vb = nb;
        na = fa;
        nb = fb;
      }
    }
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

// The token (plus one) and gate weight of each routed row: the inverse of
// dst_row, into arrays cleared to zero.
__global__ void __launch_bounds__(256) rowmap_kernel(const int32_t* __restrict__ dst_row,
                                                     const float* __restrict__ topk_w, int n, int k,
                                                     int rows, int32_t* __restrict__ row_src,
                                                     float* __restrict__ row_w) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = dst_row[i];
  if (r < 0 || r >= rows) return;  // a dropped pair
  row_src[r] = i / k + 1;
  row_w[r] = topk_w[i];
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
static size_t kpad_upper(int rows, int E, int pad) {
  return size_t(rows) + size_t(pad - 1) * E;
}

// out[e] [M][N] (fp32) = A_e^T B_e for row-major bf16 A [rows][M] and
// B [rows][N], K = rows offsets[e] .. offsets[e+1]: the weight-gradient
// schedule, without split-K (the router backward's dW_g on token chunks).
int dw_rows_bf16(const void* a, int M, const void* b, int N, const int32_t* offsets, int E,
                 int rows, float* out, hipStream_t s) {
  GemmArgs g{a, nullptr, b, nullptr, offsets, E, 0, N, rows, M,
             out, nullptr, nullptr, nullptr, nullptr, nullptr};
  return launch_gemm<CfgB, MOE_BF16, kModeDW, kSchedKR>(g, -1, s);
}

size_t grouped_bwd_ws_bytes(int rows, int h, int h_ffn, int E, int dtype) {
  (void)dtype;
  (void)h;
  (void)E;
  const size_t r = size_t(rows), hf = size_t(h_ffn);
  return al256(r * 2 * hf * 2)          // dG|dU, packed like G|U
         + al256(r * hf * 2)            // A recomputed
         + splitk_ws_bytes<CfgB>();   // split-K partial tiles
}

int grouped_bwd(const void* dyp, const void* xp, const void* h13_save, const moe_weights* W,
                const int32_t* offsets, int rows, void* dxp, float* dw1, float* dw3, float* dw2,
                void* ws, hipStream_t s) {
  const int h = W->h, hf = W->h_ffn, E = W->E;
  unsigned char* w = static_cast<unsigned char*>(ws);
  const size_t r = size_t(rows);
  void* dgu = w;
  w += al256(r * 2 * hf * 2);
  void* act = w;
  w += al256(r * hf * 2);
  void* split_ws = w;
  int rc;

  // dA = dYp W2^T, with dG, dU and A formed in the epilogue
  GemmArgs ga{dyp, nullptr, W->w2_bwd, nullptr, offsets, E, h, hf, rows, 0,
              dgu, act, const_cast<void*>(h13_save), nullptr, nullptr, nullptr};
  splitk_ws_set<CfgDA>(ga, split_ws);
  if ((rc = launch_gemm<CfgDA, MOE_BF16, kModeBwdDA, kSchedM>(ga, kTBwd1, s)))
    return rc;

  // dW2 = A^T dYp  (per expert [hf][h], fp32), K = the expert's rows of the
  // row-major A and dYp
  GemmArgs g2{act, nullptr, dyp, nullptr, offsets, E, 0, h, rows, hf,
              dw2, nullptr, nullptr, nullptr, nullptr, nullptr};
  splitk_ws_set<CfgB>(g2, split_ws);
  if ((rc = launch_gemm<CfgB, MOE_BF16, kModeDW, kSchedKR>(g2, kTBwd2, s)))
    return rc;

  // dXp = [dG|dU] W13^T
  GemmArgs g3{dgu, nullptr, W->w13_bwd, nullptr, offsets, E, 2 * hf, h, rows, 0,
              dxp, nullptr, nullptr, nullptr, nullptr, nullptr};
  splitk_ws_set<CfgB>(g3, split_ws);
  if ((rc = launch_gemm<CfgB, MOE_BF16, kModeFC2, kSchedM>(g3, kTBwd3, s)))
    return rc;

  // dW1 | dW3 = Xp^T [dG|dU]  (per expert [h][hf] each, fp32), row-major
  // operands as for dW2
  GemmArgs g4{xp, nullptr, dgu, nullptr, offsets, E, 0, 2 * hf, rows, h,
              dw1, dw3, nullptr, nullptr, nullptr, nullptr};
  splitk_ws_set<CfgB>(g4, split_ws);
  return launch_gemm<CfgB, MOE_BF16, kModeDW13, kSchedKR>(g4, kTBwd4, s);
}

}  // namespace moe_launch

namespace moe_launch {
using namespace moe;

using CfgQ = CfgFor<MOE_FP8_E4M3>::type;
// FP8 dA: 256 x 256 tiles like every other product.  FP8 accumulators live
// in VGPRs (128 per lane); with the epilogue's stores addressed by buffer
// descriptors (no 64-bit address per value) the kernel fits in 256 VGPRs
// with 8 bytes of scratch, and runs faster than on 128 x 256 tiles (waves of
// 64 x 64, which it needed while the epilogue spilled 56 VGPRs):
// DeepSeekMoE-shaped 0.836 -> 0.738 ms.
using CfgDAq = GemmCfg<2, 4, 4, 2, 1, 128, 2>;
static_assert(splitk_ws_bytes<CfgDAq>() <= splitk_ws_bytes<CfgQ>(), "one split-K area for all");

// FP8 backward workspace: bf16 dG|dU and A, dG|dU codes + row scales, the
// four transposed code blocks and their per-expert channel scales, split-K
// partials.
size_t grouped_bwd_fp8_ws_bytes(int rows, int h, int h_ffn, int E) {
  const size_t r = size_t(rows), hh = size_t(h), hf = size_t(h_ffn), e = size_t(E);
  const size_t kp = kpad_upper(rows, E, kpad_elems<MOE_FP8_E4M3>());
  return al256(r * 2 * hf * 2) + al256(r * hf * 2) + al256(r * 2 * hf) + al256(r * 4) +
         2 * al256(hh * kp) + al256(hf * kp) + al256(2 * hf * kp) +
         2 * al256(e * hh * 4) + al256(e * 3 * hf * 4) + 2 * al256(r * 4) + splitk_ws_bytes<CfgQ>();
}

static int xpose_q(const void* src, int C, const int32_t* offsets, int E, int rows, void* dst,
                   float* scale, bool have_amax, hipStream_t s, const int32_t* row_src = nullptr,
                   const float* row_w = nullptr, int ntok = 0) {
  if (C % 64 != 0) return MOE_ERR_SHAPE;
  // Workgroups per CU: as many as keep the strips of the items in progress
  // (128 bytes per row of the expert, read twice) within ~192 MiB, so the
  // encoding pass finds them in the 256 MB Infinity Cache; at least 4 to keep
  // enough loads in flight, at most 8 (the occupancy the kernel reaches).
  // DeepSeekMoE-shaped FP8 step (1536 rows per expert): 4 per CU, the four
  // transposes 0.95 -> 0.86 ms; with 6-8 per CU the strips no longer fit and
  // with 3 or fewer the loads in flight fall short (both 0.95 ms).
  const int items = (C / 64) * E;
  const double strip = 128.0 * (double(rows) / (E > 0 ? E : 1) + 1.0);
  int per_cu = int((192.0 * 1024 * 1024) / (double(num_cus()) * strip));
  per_cu = per_cu < 4 ? 4 : (per_cu > 8 ? 8 : per_cu);
  // one pass, or gathered rows of a token-major source the Infinity Cache holds
  // whole: nothing to bound
  if (have_amax || row_src) per_cu = 8;
  const int grid = items < num_cus() * per_cu ? items : num_cus() * per_cu;
  if (grid <= 0) return MOE_OK;
  hipLaunchKernelGGL(xpose_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t*)src, C,
                     offsets, E, rows, kpad_elems<MOE_FP8_E4M3>(), dst, scale, int(have_amax), row_src,
                     row_w, ntok);
  return launch_status();
}

// With dst_row, dyp and xp are the token-major dY and x ([T][h]) and the
// weight-gradient operands are gathered from them (topk_w weighting dY).
int grouped_bwd_fp8(const void* dyp_q, const float* dyp_scale, const void* dyp, const void* xp,
                    const void* h13_save, const moe_weights* W, const int32_t* offsets, int rows,
                    void* dxp, float* dw1, float* dw3, float* dw2, void* ws, hipStream_t s,
                    const int32_t* dst_row, const float* topk_w, int T, int k) {
  const int h = W->h, hf = W->h_ffn, E = W->E;
  const size_t r = size_t(rows), kp = kpad_upper(rows, E, kpad_elems<MOE_FP8_E4M3>());
  unsigned char* w = static_cast<unsigned char*>(ws);
  auto take = [&](size_t bytes) { unsigned char* p = w; w += al256(bytes); return p; };
  void* dgu = take(r * 2 * hf * 2);
  void* act = take(r * hf * 2);
  void* dgu_q = take(r * 2 * hf);
  float* dgu_s = reinterpret_cast<float*>(take(r * 4));
  void* xpT = take(size_t(h) * kp);
  void* dypT = take(size_t(h) * kp);
  void* actT = take(size_t(hf) * kp);
  void* dguT = take(2 * size_t(hf) * kp);
  float* sx = reinterpret_cast<float*>(take(size_t(E) * h * 4));
  float* sd = reinterpret_cast<float*>(take(size_t(E) * h * 4));
  // A's channel scales, then dG|dU's: one array, which the dA epilogue fills
  // with the column maxima first
  float* sa = reinterpret_cast<float*>(take(size_t(E) * 3 * hf * 4));
  float* sg = sa + size_t(E) * hf;
  int32_t* row_src = reinterpret_cast<int32_t*>(take(r * 4));
  float* row_w = reinterpret_cast<float*>(take(r * 4));
  void* split_ws = w;
  int rc;
  if (dst_row == nullptr) {
    row_src = nullptr;
    row_w = nullptr;
  } else if (rows > 0) {
    hipLaunchKernelGGL(zero_u32_kernel<0>, dim3(ceil_div(rows, 256)), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(row_src), rows);
    hipLaunchKernelGGL(rowmap_kernel, dim3(ceil_div(T * k, 256)), dim3(256), 0, s, dst_row, topk_w,
                       T * k, k, rows, row_src, row_w);
  }

  timer_begin(kTXpose, s);
  if ((rc = xpose_q(xp, h, offsets, E, rows, xpT, sx, false, s, row_src, nullptr, T))) return rc;
  if ((rc = xpose_q(dyp, h, offsets, E, rows, dypT, sd, false, s, row_src, row_w, T))) return rc;
  {
    const int n = E * 3 * hf;  // the column maxima start from zero
    hipLaunchKernelGGL(zero_u32_kernel<0>, dim3(ceil_div(n, 256)), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(sa), n);
  }
  timer_end(kTXpose, s);

  // dA = dYp W2^T on FP8 codes; epilogue rescales, forms dG, dU and A and
  // takes their column maxima per expert
  GemmArgs ga{dyp_q, dyp_scale, W->w2_bwd, W->w2_bwd_scale, offsets, E, h, hf, rows, 0,
              dgu, act, const_cast<void*>(h13_save), sa, nullptr, nullptr};
  splitk_ws_set<CfgDAq>(ga, split_ws);
  if ((rc = launch_gemm<CfgDAq, MOE_FP8_E4M3, kModeBwdDA, kSchedM>(ga, kTBwd1, s))) return rc;

  timer_begin(kTQuant, s);
  if (rows > 0)  // no rows: the weight gradients below are still written (as zeros)
    hipLaunchKernelGGL(rowq_kernel, dim3(ceil_div(rows, 4)), dim3(256), 0, s, (const uint16_t*)dgu,
                       rows, 2 * hf, (uint8_t*)dgu_q, dgu_s);
  timer_end(kTQuant, s);
  timer_begin(kTXpose, s);
  if ((rc = xpose_q(act, hf, offsets, E, rows, actT, sa, true, s))) return rc;
  if ((rc = xpose_q(dgu, 2 * hf, offsets, E, rows, dguT, sg, true, s))) return rc;
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
