// Forward GroupedGEMM of the SwiGLU experts over expert-contiguous rows.
//
// One kernel runs every expert's matrix products (MegaScale-MoE research
// digest §3.3: a GroupedGEMM runs several experts' products in one kernel;
// paper review §三 training flow "专家计算").  Each expert is a SwiGLU FFN
// with three h x h_ffn matrices, FC1 then FC2 (review §三 core formulas and
// §四 selective recomputation).  Per-token FP8 scales (review §三
// compression layer, §四 FP8 row) enter as a rank-1 rescale in the epilogue.
//
// gfx950 design
//   * Both operands are K-contiguous ("NT"): routed rows [rows][K] and packed
//     weights [E][N][K], so every 16-byte global load and LDS read feeds an
//     MFMA operand directly.
//   * Tile 256 x 256, 128 bytes of K per stage (64 bf16, 32 fp32, 128 fp8),
//     eight waves of 128 x 64 (4 x 2 MFMA 32x32 blocks, 128 fp32 accumulators
//     per lane), two per SIMD so that one can issue MFMAs while the other
//     waits on a load.  Two LDS stages (128 KB) give one barrier per K step.  Operands go global -> LDS directly (buffer_load ... lds, no
//     VGPR staging); the next slab's loads are in flight while the current
//     one computes, and the next slab's first fragments are read right after
//     the barrier while the last substep's MFMAs still run.
//   * LDS rows are 128 B with the 16-byte chunk index XOR-swizzled by
//     (row/2)%8, so the 64 lanes of an operand read hit distinct banks.
//   * Persistent: one workgroup per CU walks a tile list built on device from
//     `offsets` (no host round trip for the ragged per-expert sizes).  Tiles
//     are ordered expert by expert, m-tiles fastest, and workgroup ids are
//     remapped so the 32 workgroups of one XCD take 32 consecutive tiles:
//     they share A row blocks and weight column blocks in that XCD's L2.
//   * FC1's packed weight interleaves 32 gate and 32 up channels, so a wave
//     holds G and U of the same channels in registers: SwiGLU is applied in
//     the epilogue and only A = SiLU(G)*U (and optionally G|U) is written.
#include "gemm_engine.h"

namespace moe {

// FP8: act (fp32) -> E4M3 codes with per-row scale amax/448; amax is the max
// of the row's ntn per-column-tile maxima that FC1's epilogue stored.
__global__ void __launch_bounds__(256) quant_act_kernel(const float* __restrict__ act,
                                                        const float* __restrict__ row_amax, int ntn,
                                                        const int32_t* __restrict__ offsets,
                                                        int E, int hf, uint8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= offsets[E]) return;
  float amax = 0.f;
  for (int j = lane; j < ntn; j += 64) amax = fmaxf(amax, row_amax[size_t(row) * ntn + j]);
  amax = wave_max(amax);
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (lane == 0) scale[row] = s;
  const QuotScale qs = quot_scale(s);
  const f32x4* src = reinterpret_cast<const f32x4*>(act + size_t(row) * hf);
  uint32_t* dst = reinterpret_cast<uint32_t*>(q + size_t(row) * hf);
  constexpr int kBatch = 8;  // 16-byte loads per lane in flight
  const int n4 = hf / 4;
  for (int c0 = lane; c0 < n4; c0 += 64 * kBatch) {
    f32x4 v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (c0 + 64 * b < n4) v[b] = src[c0 + 64 * b];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (c0 + 64 * b >= n4) break;
      dst[c0 + 64 * b] = e4m3x4_quot(v[b][0], v[b][1], v[b][2], v[b][3], qs);
    }
  }
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// FC1's column tiles (packed G|U, 2 h_ffn wide): one row-maximum slot each.
static size_t fc1_col_tiles(int h_ffn) {
  constexpr int BN = CfgFor<MOE_FP8_E4M3>::type::kBN;
  return size_t((2 * h_ffn + BN - 1) / BN);
}

size_t grouped_fwd_ws_bytes(int rows, int h, int h_ffn, int E, int dtype) {
  (void)h; (void)E;
  size_t r = size_t(rows), hf = size_t(h_ffn);
  size_t act = al256(r * hf * (dtype == MOE_BF16 ? 2 : 4));
  if (dtype == MOE_FP8_E4M3) act += al256(r * hf) + al256(r * 4 * fc1_col_tiles(h_ffn)) + al256(r * 4);
  return act + splitk_ws_bytes<CfgFor<MOE_BF16>::type>();
}

template <int DT, int MODE>
static int launch_fwd_gemm(const GemmArgs& a, hipStream_t s) {
  return launch_gemm<typename CfgFor<DT>::type, DT, MODE, kSchedM>(a, MODE == kModeFC1 ? kTFc1 : kTFc2, s);
}

template <int DT>
static int fwd_typed(const void* xp, const float* xp_scale, const moe_weights* W,
                     const int32_t* offsets, int rows, void* h13_save, void* yp, int yp_f32,
                     void* ws, hipStream_t s) {
  const int h = W->h, hf = W->h_ffn, E = W->E;
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* act = w;
  size_t act_b = al256(size_t(rows) * hf * (DT == MOE_BF16 ? 2 : 4));
  const size_t ntn = fc1_col_tiles(hf);
  const size_t amax_b = al256(size_t(rows) * 4 * ntn);
  void* split_ws = w + act_b + (DT == MOE_FP8_E4M3 ? al256(size_t(rows) * hf) + amax_b + al256(size_t(rows) * 4) : 0);
  uint8_t* actq = nullptr;
  float* amax = nullptr;
  float* ascale = nullptr;
  if (DT == MOE_FP8_E4M3) {
    actq = reinterpret_cast<uint8_t*>(w + act_b);
    amax = reinterpret_cast<float*>(w + act_b + al256(size_t(rows) * hf));
    ascale = reinterpret_cast<float*>(w + act_b + al256(size_t(rows) * hf) + amax_b);
  }
  GemmArgs a1{xp, xp_scale, W->w13, W->w13_scale, offsets, E, h, 2 * hf, rows, 0,
              act, nullptr, h13_save, amax, nullptr, nullptr};
  splitk_ws_set<typename CfgFor<DT>::type>(a1, split_ws);
  int rc = launch_fwd_gemm<DT, kModeFC1>(a1, s);
  if (rc) return rc;
  if (DT == MOE_FP8_E4M3) {
    timer_begin(kTQuant, s);
    hipLaunchKernelGGL(quant_act_kernel, dim3(ceil_div(rows, 4)), dim3(256), 0, s,
                       (const float*)act, amax, int(ntn), offsets, E, hf, actq, ascale);
    timer_end(kTQuant, s);
    GemmArgs a2{actq, ascale, W->w2, W->w2_scale, offsets, E, hf, h, rows, 0, yp, nullptr, nullptr, nullptr,
                nullptr, nullptr, yp_f32};
    splitk_ws_set<typename CfgFor<DT>::type>(a2, split_ws);
    return launch_fwd_gemm<DT, kModeFC2>(a2, s);
  }
  GemmArgs a2{act, nullptr, W->w2, nullptr, offsets, E, hf, h, rows, 0, yp, nullptr, nullptr, nullptr,
              nullptr, nullptr, yp_f32};
  splitk_ws_set<typename CfgFor<DT>::type>(a2, split_ws);
  return launch_fwd_gemm<DT, kModeFC2>(a2, s);
}

int grouped_fwd(const void* xp, const float* xp_scale, const moe_weights* W,
                const int32_t* offsets, int rows, void* h13_save, void* yp, int yp_dtype, void* ws,
                hipStream_t s) {
  if (rows == 0) return MOE_OK;
  const int f = yp_dtype == MOE_F32;
  switch (W->dtype) {
    case MOE_F32: return fwd_typed<MOE_F32>(xp, xp_scale, W, offsets, rows, h13_save, yp, 1, ws, s);
    case MOE_BF16: return fwd_typed<MOE_BF16>(xp, xp_scale, W, offsets, rows, h13_save, yp, f, ws, s);
    case MOE_FP8_E4M3:
      return fwd_typed<MOE_FP8_E4M3>(xp, xp_scale, W, offsets, rows, h13_save, yp, f, ws, s);
  }
  return MOE_ERR_DTYPE;
}

}  // namespace moe_launch
