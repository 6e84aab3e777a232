// Router backward and the load-balance loss.
//
// The gating network is trainable (MegaScale-MoE paper review, §三 MoE layer
// structure), so W_g and the router bias receive gradients through the gate
// weights of the combine.  Load balance uses an auxiliary loss (research
// digest §3.2, discussion of Figure 7, which points to DeepSeek-V2); the pages print
// no formula, and the expert-level balance loss of DeepSeek-V2 is used:
//     L_aux = alpha * sum_e f_e P_e,   f_e = E/(kT) * count_e,
//     P_e   = (1/T) sum_t softmax(L_t)_e.
// The top-k selection is piecewise constant in the logits and held fixed.
//
// Kernels (every sum over tokens is taken in a fixed order, so results are
// deterministic):
//   dlogits   one wave per token: dw_j = <dY_t, Yp[dst_row_tj]>, the top-k
//             softmax backward, the aux-loss gradient, dL_t written in fp32;
//   dwg       dW_g = x^T dL: with bf16 x on the GroupedGEMM's weight-gradient
//             schedule, dL split into two bf16 parts and the tokens in chunks
//             (see rbwd_dl_split_kernel); with fp32 x, partials over 128-token
//             chunks on fp32 MFMA (64 columns x 64 experts per pass); then the
//             chunks are added in order (and the bias gradient, the column
//             sums of dL);
//   dx        dx = dx_in + dL W_g^T, 32 tokens per workgroup: with a bf16 W_g
//             and E <= 64 on bf16 MFMA with dL split into two bf16 parts,
//             else on fp32 MFMA with the dL rows in LDS;
//   aux       per-workgroup column sums of softmax(L_t), then one workgroup
//             adds them in order and forms the loss.
#include "common.h"

namespace moe {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <bool kF32>
__device__ __forceinline__ void load8(const void* base, size_t elem, float* f) {
  if (kF32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
  } else {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[i]); f[2 * i + 1] = bf16_hi(v[i]); }
  }
}

// 8 values from one (bf16) or two (fp32) 16-byte words.
template <bool kF32>
__device__ __forceinline__ void unpack8f(const u32x4 (&v)[kF32 ? 2 : 1], float* f) {
  if (kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = __uint_as_float(v[0][i]); f[4 + i] = __uint_as_float(v[kF32 ? 1 : 0][i]); }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[0][i]); f[2 * i + 1] = bf16_hi(v[0][i]); }
  }
}

template <bool kF32>
__device__ __forceinline__ float load1(const void* base, size_t elem) {
  return kF32 ? static_cast<const float*>(base)[elem]
              : bf16_to_f32(static_cast<const uint16_t*>(base)[elem]);
}

// rows x 64 fp32 tile [r][e] of a row-major [*][E] fp32 array (rows r0.., experts
// e0..e0+63) into LDS with row pitch `pitch`, zero outside (rows >= nr or
// experts >= ne).  Every thread issues all its 16-byte loads before its first
// LDS store, so the loads overlap.
template <int ROWS>
__device__ __forceinline__ void stage_tile64(const float* __restrict__ src, int E, int r0, int nr,
                                             int e0, int ne, float* lds, int pitch) {
  constexpr int PER = ROWS * 16 / 256;  // f32x4 per thread
  static_assert(PER * 256 == ROWS * 16, "whole f32x4 per thread");
  const bool vec = (E & 3) == 0;
  f32x4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = threadIdx.x + 256 * i, r = q >> 4, e = (q & 15) * 4;
    v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r < nr) {
      const float* row = src + size_t(r0 + r) * E + e0 + e;
      if (vec && e + 4 <= ne) {
        v[i] = *reinterpret_cast<const f32x4*>(row);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e + j < ne) v[i][j] = row[j];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = threadIdx.x + 256 * i, r = q >> 4, e = (q & 15) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds[r * pitch + e + j] = v[i][j];
  }
}

// dL for one token per wave.  KM bounds k (all slots' dots run together).
// kF32: dY is fp32 (else bf16); kYF32: the expert outputs Yp are fp32.
template <bool kF32, bool kYF32, int KM>
__global__ void __launch_bounds__(256) rbwd_dlogits_kernel(
    const void* __restrict__ dy, const void* __restrict__ yp, const int32_t* __restrict__ dst_row,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const float* __restrict__ logits, const int32_t* __restrict__ counts, int T, int h, int E,
    int k, float alpha, float* __restrict__ dL) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (E == 1) {
    // one expert: the top-1 weight is 1 and the balance loss constant, so
    // dL is exactly zero (the sums below would leave rounding noise)
    if (lane == 0) dL[t] = 0.f;
    return;
  }
  int rows[KM];
  float wt[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    rows[j] = -1;
    wt[j] = 0.f;
    if (j < k) {
      const int r = dst_row[size_t(t) * k + j];
      rows[j] = (r < 0 || r >= T * k) ? -1 : r;
      wt[j] = topk_w[size_t(t) * k + j];
    }
  }
  // dw_j = <dY_t, Yp_j>: lanes take 8-element chunks, then a butterfly sum.
  // A batch of kB chunk positions has all its loads (dY and every routed
  // row) issued before the first multiply; this is the last read of both,
  // so the loads are nontemporal.
  constexpr int kB = KM <= 2 ? 8 : (KM <= 4 ? 4 : (KM <= 8 ? 2 : 1));
  constexpr int kVec = kF32 ? 2 : 1;  // 16-byte loads per 8 elements of dY
  constexpr int kVecY = kYF32 ? 2 : 1;  // and of Yp
  const size_t esz = kF32 ? 4 : 2, eszy = kYF32 ? 4 : 2;
  float part[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) part[j] = 0.f;
  for (int c0 = lane * 8; c0 < h; c0 += 64 * 8 * kB) {
    u32x4 dv[kB][kVec], yv[kB][KM][kVecY];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int c = c0 + 512 * b;
#pragma unroll
      for (int q = 0; q < kVec; ++q) {
        dv[b][q] = u32x4{0, 0, 0, 0};
        if (c < h)
          dv[b][q] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(static_cast<const char*>(dy) + (size_t(t) * h + c) * esz) + q);
      }
#pragma unroll
      for (int j = 0; j < KM; ++j)
#pragma unroll
        for (int q = 0; q < kVecY; ++q) {
          yv[b][j][q] = u32x4{0, 0, 0, 0};
          if (c < h && rows[j] >= 0)
            yv[b][j][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                static_cast<const char*>(yp) + (size_t(rows[j]) * h + c) * eszy) + q);
        }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      float d[8];
      unpack8f<kF32>(dv[b], d);
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        float y[8];
        unpack8f<kYF32>(yv[b][j], y);
#pragma unroll
        for (int i = 0; i < 8; ++i) part[j] = fmaf(d[i], y[i], part[j]);
      }
    }
  }
  float inner = 0.f;
  float dwt[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    dwt[j] = wave_sum(part[j]);
    inner += wt[j] * dwt[j];
  }
  // aux loss: s_t = softmax(L_t), g_e = alpha f_e / T
  const float* L = logits + size_t(t) * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, L[e]);
  m = wave_max(m);
  float z = 0.f, zg = 0.f;
  const float gs = alpha * float(E) / (float(k) * float(T) * float(T));
  for (int e = lane; e < E; e += 64) {
    const float p = __expf(L[e] - m);
    z += p;
    zg += p * gs * float(counts[e]);
  }
  z = wave_sum(z);
  zg = wave_sum(zg);
  const float inv = 1.0f / z, sg = zg * inv;
  for (int e = lane; e < E; e += 64) {
    float v = 0.f;
    if (alpha != 0.f) {
      const float s = __expf(L[e] - m) * inv;
      v = s * (gs * float(counts[e]) - sg);
    }
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k && topk_idx[size_t(t) * k + j] == e) v += wt[j] * (dwt[j] - inner);
    dL[size_t(t) * E + e] = v;
  }
}

constexpr int kDwCols = 64;   // x columns per dW_g workgroup
constexpr int kDwEC = 64;     // experts per pass
constexpr int kDwTC = 128;    // tokens per chunk
constexpr int kDwPad = 65;    // fp32 per LDS row (one bank of padding)

// partial[chunk][e][c] = sum over the chunk's tokens of x[t][c] dL[t][e], on
// fp32 MFMA 32x32x2 with K = tokens: wave w owns expert block w%2 and column
// block w/2 of the 64 x 64 (experts x columns) pass.  The chunk's dL slice
// and x tile are staged in LDS as fp32 ([token][expert], [token][column]).
template <bool kF32>
__global__ void __launch_bounds__(256) rbwd_dwg_kernel(const void* __restrict__ x,
                                                       const float* __restrict__ dL, int T, int h,
                                                       int E, float* __restrict__ part,
                                                       float* __restrict__ part_b) {
  __shared__ float dls[kDwTC * kDwPad];
  __shared__ float xs[kDwTC * kDwPad];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int mb = wave & 1, nb = wave >> 1;
  const int c0 = blockIdx.x * kDwCols;
  const int t0 = blockIdx.y * kDwTC;
  const int nt = T - t0 < kDwTC ? T - t0 : kDwTC;
  {  // x tile: 128 tokens x 64 columns in 8-column groups, loads first
    constexpr int PER = kDwTC * 8 / 256;
    float f[PER][8];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + 256 * i, tt = q >> 3, g8 = (q & 7) * 8;
      if (tt < nt) {
        load8<kF32>(x, size_t(t0 + tt) * h + c0 + g8, f[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[i][j] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + 256 * i, tt = q >> 3, g8 = (q & 7) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[tt * kDwPad + g8 + j] = f[i][j];
    }
  }
  for (int e0 = 0; e0 < E; e0 += kDwEC) {
    const int ne = E - e0 < kDwEC ? E - e0 : kDwEC;
    __syncthreads();  // previous pass done with dls (and the x tile staged)
    stage_tile64<kDwTC>(dL, E, t0, nt, e0, ne, dls, kDwPad);
    __syncthreads();
    if (32 * mb < ne) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const float* ap = dls + half * kDwPad + 32 * mb + l32;  // A[m = expert][k = token]
      const float* bp = xs + half * kDwPad + 32 * nb + l32;   // B[k = token][n = column]
#pragma unroll 8
      for (int kk = 0; kk < kDwTC; kk += 2)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ap[kk * kDwPad], bp[kk * kDwPad], acc, 0, 0, 0);
      // C: row (expert) 8(r/4) + 4 half + r%4, column l32
      const int col = c0 + 32 * nb + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = 32 * mb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (e < ne) part[(size_t(blockIdx.y) * E + e0 + e) * h + col] = acc[r];
      }
    }
    // bias gradient: column sums of dL over the chunk, by the first column block
    if (blockIdx.x == 0 && tid < ne) {
      float v = 0.f;
      for (int tt = 0; tt < nt; ++tt) v += dls[tt * kDwPad + tid];
      part_b[size_t(blockIdx.y) * E + e0 + tid] = v;
    }
  }
}

// dw_gate[c][e] = sum over chunks (in order) of partial[chunk][e][c]; dbias
// likewise from the per-chunk column sums.
__global__ void __launch_bounds__(256) rbwd_dwg_reduce_kernel(const float* __restrict__ part,
                                                              const float* __restrict__ part_b,
                                                              int nchunk, int h, int E,
                                                              float* __restrict__ dw_gate,
                                                              float* __restrict__ dbias) {
  const size_t n = size_t(h) * E;
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) {
    // loads in batches of 8, adds in chunk order
    float v = 0.f;
    int q = 0;
    for (; q + 8 <= nchunk; q += 8) {
      float b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = part[size_t(q + j) * n + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) v += b[j];
    }
    for (; q < nchunk; ++q) v += part[size_t(q) * n + i];
    const size_t e = i / h, c = i - e * h;  // i indexes [e][c]
    dw_gate[c * E + e] = v;
  }
  if (dbias && i < size_t(E)) {
    float v = 0.f;
    for (int q = 0; q < nchunk; ++q) v += part_b[size_t(q) * E + i];
    dbias[i] = v;
  }
}

// BF16 x: dW_g = x^T dL runs on the GroupedGEMM's weight-gradient schedule
// (bf16 MFMA, row-major operands read through the LDS transpose read), with
// the tokens cut into `nch` chunks that act as its experts, so the chunks'
// products run side by side; dL enters as two bf16 parts (hi = bf16(dL),
// lo = bf16(dL - hi), side by side in rows of E2 = 2E rounded up to 8
// values; the pad columns are never read back), which carries it to ~2^-17
// relative with fp32 sums.  Blocks [0, nconv) write the two parts (block 0
// also the chunk boundaries); with dbias, block nconv + e sums column e of dL
// in fp32 (thread j over tokens j, j + 256, ... in order, then the 256
// partials in order).
__global__ void __launch_bounds__(256) rbwd_dl_split_kernel(const float* __restrict__ dL, int T,
                                                            int E, int E2, int chunk, int nch,
                                                            int nconv,
                                                            uint16_t* __restrict__ dlhl,
                                                            int32_t* __restrict__ choff,
                                                            float* __restrict__ dbias) {
  const int tid = threadIdx.x;
  if (int(blockIdx.x) < nconv) {
    if (blockIdx.x == 0)
      for (int q = tid; q <= nch; q += 256) choff[q] = int64_t(q) * chunk < T ? q * chunk : T;
    const size_t n = size_t(T) * E;
    for (size_t q = size_t(blockIdx.x) * 256 + tid; q < n; q += size_t(nconv) * 256) {
      const size_t t = q / E, e = q - t * E;
      const float v = dL[q];
      const uint32_t hb = f32_to_bf16_bits(v);
      uint16_t* row = dlhl + t * E2;
      row[e] = uint16_t(hb);
      row[E + e] = uint16_t(f32_to_bf16_bits(v - __uint_as_float(hb << 16)));
    }
    return;
  }
  __shared__ float ps[256];
  const int e = blockIdx.x - nconv;
  float v = 0.f;
  for (int t0 = tid; t0 < T; t0 += 256 * 8) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = t0 + 256 * i;
      a[i] = t < T ? dL[size_t(t) * E + e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v += a[i];
  }
  ps[tid] = v;
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
    for (int j = 0; j < 256; ++j) sum += ps[j];
    dbias[e] = sum;
  }
}

// dw_gate[c][e] = sum over chunks (in order) of P[ch][c][e] + P[ch][c][E + e]
// (the products of the two parts of dL).
__global__ void __launch_bounds__(256) rbwd_dwg_gemm_reduce_kernel(const float* __restrict__ P,
                                                                   int nch, int h, int E, int E2,
                                                                   float* __restrict__ dw_gate) {
  const size_t n = size_t(h) * E, pitch = size_t(h) * E2;
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;  // [c][e]
  if (i >= n) return;
  const size_t c = i / E, e = i - c * E;
  const float* p = P + c * E2 + e;
  float v = 0.f;
  int q = 0;
  for (; q + 4 <= nch; q += 4) {
    float a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { a[j] = p[size_t(q + j) * pitch]; b[j] = p[size_t(q + j) * pitch + E]; }
#pragma unroll
    for (int j = 0; j < 4; ++j) v += a[j] + b[j];
  }
  for (; q < nch; ++q) v += p[size_t(q) * pitch] + p[size_t(q) * pitch + E];
  dw_gate[i] = v;
}

constexpr int kDxTokens = 32;
constexpr int kDxEC = 64;           // experts per pass
constexpr int kDxPad = kDxEC + 1;   // fp32 per LDS row
constexpr int kDxCbPer = 16;        // 32-column blocks per workgroup (4 per wave)

// dx[t][c] = dx_in[t][c] + sum_e dL[t][e] W_g[c][e] on fp32 MFMA 32x32x2 with
// K = experts: 32 tokens per workgroup, their dL rows in LDS (A operand);
// each wave takes 32-column blocks in turn, every lane holding a 32-expert
// segment of its column's W_g row in registers (B operand).  With E <= 64 the
// dL rows are staged once and the column loop runs without barriers.
template <bool kF32>
__global__ void __launch_bounds__(256) rbwd_dx_kernel(const float* __restrict__ dL,
                                                      const void* __restrict__ wg,
                                                      const float* __restrict__ dx_in, int T,
                                                      int h, int E, void* __restrict__ dx) {
  __shared__ float dls[kDxTokens * kDxPad];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int t0 = blockIdx.x * kDxTokens;
  const int nt = T - t0 < kDxTokens ? T - t0 : kDxTokens;
  const int ncb = h / 32;
  const bool vec = (E & 7) == 0;
  const int nchunks = (E + kDxEC - 1) / kDxEC;
  auto stage = [&](int e0, int ne) { stage_tile64<kDxTokens>(dL, E, t0, nt, e0, ne, dls, kDxPad); };
  if (nchunks == 1) {
    stage(0, E);
    __syncthreads();
  }
  const float* ap = dls + l32 * kDxPad;  // A[m = token][k = expert]
  // workgroup y takes column blocks y*kDxCbPer .. ; every wave runs the same
  // number of rounds
  const int cb0 = blockIdx.y * kDxCbPer;
  const int cbn = ncb - cb0 < kDxCbPer ? ncb - cb0 : kDxCbPer;
  const int rounds = (cbn + 3) / 4;
  for (int rd = 0; rd < rounds; ++rd) {
    const int cb = cb0 + rd * 4 + wave;
    const bool active = cb < cb0 + cbn;
    const int c = cb * 32 + l32;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    for (int ch = 0; ch < nchunks; ++ch) {
      const int e0 = ch * kDxEC, ne = E - e0 < kDxEC ? E - e0 : kDxEC;
      if (nchunks > 1) {
        __syncthreads();
        stage(e0, ne);
        __syncthreads();
      }
      if (!active) continue;
      // K order: at step s the two halves of the wave take experts 32 half + s,
      // so each lane holds one contiguous 32-expert segment of its W_g row
      float wv[32];
      const int eh = e0 + 32 * half;
      if (vec) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float f[8];
          if (32 * half + 8 * g < ne) {
            load8<kF32>(wg, size_t(c) * E + eh + 8 * g, f);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = 0.f;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) wv[8 * g + i] = f[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          wv[i] = 32 * half + i < ne ? load1<kF32>(wg, size_t(c) * E + eh + i) : 0.f;
      }
      const float* ah = ap + 32 * half;
#pragma unroll
      for (int i = 0; i < 32; ++i)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ah[i], wv[i], acc, 0, 0, 0);
    }
    if (active) {
      // C: row (token) 8(r/4) + 4 half + r%4, column l32
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tt = 8 * (r >> 2) + 4 * half + (r & 3);
        if (tt < nt) {
          const size_t o = size_t(t0 + tt) * h + c;
          const float v = (dx_in ? dx_in[o] : 0.f) + acc[r];
          if (kF32) static_cast<float*>(dx)[o] = v;
          else static_cast<uint16_t*>(dx)[o] = uint16_t(f32_to_bf16_bits(v));
        }
      }
    }
  }
}

// BF16 W_g with E <= 64: the same dx on bf16 MFMA 32x32x16.  dL is split
// into hi = bf16(dL) and lo = bf16(dL - hi), and both parts multiply the
// (exact) bf16 W_g with fp32 accumulation, which carries dL to ~2^-17
// relative, at an eighth of the fp32 MFMA's issue time.  32 tokens per
// workgroup: every lane keeps its token's dL fragments (hi and lo) in
// registers; each wave takes 32-column blocks in turn, loads the block's
// dx_in (its last read: nontemporal) before its MFMAs and stores the sum as
// bf16.
template <int KC>  // K steps of 16 experts, KC = ceil(E / 16) <= 4
__global__ void __launch_bounds__(256) rbwd_dx_bf16_kernel(const float* __restrict__ dL,
                                                           const uint16_t* __restrict__ wg,
                                                           const float* __restrict__ dx_in, int T,
                                                           int h, int E, uint16_t* __restrict__ dx) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int t0 = blockIdx.x * kDxTokens;
  const int nt = T - t0 < kDxTokens ? T - t0 : kDxTokens;
  // A fragments: token l32 (rows past the batch read token t0, never stored),
  // experts 16 s + 8 half + i
  const float* dlr = dL + size_t(t0 + (l32 < nt ? l32 : 0)) * E;
  u32x4 ahi[KC], alo[KC];
#pragma unroll
  for (int st = 0; st < KC; ++st) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 16 * st + 8 * half + i;
      v[i] = e < E ? dlr[e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h0 = f32_to_bf16_bits(v[2 * i]), h1 = f32_to_bf16_bits(v[2 * i + 1]);
      ahi[st][i] = h0 | (h1 << 16);
      alo[st][i] = pack_bf16x2(v[2 * i] - __uint_as_float(h0 << 16), v[2 * i + 1] - __uint_as_float(h1 << 16));
    }
  }
  const bool vec = (E & 7) == 0;
  const int ncb = h / 32;
  const int cb0 = blockIdx.y * kDxCbPer;
  const int cbe = ncb < cb0 + kDxCbPer ? ncb : cb0 + kDxCbPer;
  for (int cb = cb0 + wave; cb < cbe; cb += 4) {
    const int c = cb * 32 + l32;
    // C: row (token) 8(r/4) + 4 half + r%4, column l32
    float din[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = 8 * (r >> 2) + 4 * half + (r & 3);
      din[r] = (dx_in && tt < nt) ? __builtin_nontemporal_load(dx_in + size_t(t0 + tt) * h + c)
                                  : 0.f;
    }
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const uint16_t* wr = wg + size_t(c) * E;
#pragma unroll
    for (int st = 0; st < KC; ++st) {
      const int e0 = 16 * st + 8 * half;
      u32x4 b = u32x4{0, 0, 0, 0};
      if (vec) {
        if (e0 < E) b = *reinterpret_cast<const u32x4*>(wr + e0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = e0 + 2 * i < E ? wr[e0 + 2 * i] : 0u;
          const uint32_t hi = e0 + 2 * i + 1 < E ? wr[e0 + 2 * i + 1] : 0u;
          b[i] = lo | (hi << 16);
        }
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ahi[st]),
                                                    __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, alo[st]),
                                                    __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = 8 * (r >> 2) + 4 * half + (r & 3);
      if (tt < nt) dx[size_t(t0 + tt) * h + c] = uint16_t(f32_to_bf16_bits(din[r] + acc[r]));
    }
  }
}

constexpr int kAuxTokens = 64;  // tokens per aux workgroup

// colsum[b][e] = sum over the workgroup's 64 tokens (in token order) of
// softmax(L_t)_e: thread t forms its token's probabilities in LDS, then
// thread e adds its column.
__global__ void __launch_bounds__(256) aux_colsum_kernel(const float* __restrict__ logits, int T,
                                                         int E, float* __restrict__ colsum) {
  extern __shared__ __align__(16) float sm[];  // [64][E]
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kAuxTokens;
  const int nt = T - t0 < kAuxTokens ? T - t0 : kAuxTokens;
  if (tid < nt) {
    const float* L = logits + size_t(t0 + tid) * E;
    float* p = sm + size_t(tid) * E;
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, L[e]);
    float z = 0.f;
    for (int e = 0; e < E; ++e) {
      const float v = __expf(L[e] - m);
      p[e] = v;
      z += v;
    }
    const float inv = 1.0f / z;
    for (int e = 0; e < E; ++e) p[e] *= inv;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float v = 0.f;
    for (int tt = 0; tt < nt; ++tt) v += sm[size_t(tt) * E + e];
    colsum[size_t(blockIdx.x) * E + e] = v;
  }
}

__global__ void __launch_bounds__(256) aux_loss_kernel(const float* __restrict__ colsum, int nblk,
                                                       const int32_t* __restrict__ counts, int T,
                                                       int E, int k, float alpha,
                                                       float* __restrict__ loss) {
  __shared__ float terms[MOE_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += 256) {
    // loads in batches of 8, adds in workgroup order
    float p = 0.f;
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = colsum[size_t(b + j) * E + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) p += v[j];
    }
    for (; b < nblk; ++b) p += colsum[size_t(b) * E + e];
    const float f = float(E) / (float(k) * float(T)) * float(counts[e]);
    terms[e] = f * (p / float(T));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int e = 0; e < E; ++e) s += terms[e];
    loss[0] = alpha * s;
  }
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// Token chunks of the BF16 dW_g product: about one persistent round of
// GEMM tiles (256) over ceil(h/256) x ceil(E2/256) tiles per chunk; chunks
// are whole 64-row slabs except the last.  E2 = 2E rounded up to 8.
static int dwg_e2(int E) { return (2 * E + 7) / 8 * 8; }
static void dwg_chunks(int T, int h, int E, int* chunk, int* nch) {
  const int tiles = ceil_div(h, 256) * ceil_div(dwg_e2(E), 256);
  int n = 256 / tiles > 1 ? 256 / tiles : 1;
  int c = ceil_div(ceil_div(T, n), 64) * 64;
  *chunk = c;
  *nch = ceil_div(T, c);
}

size_t router_bwd_ws_bytes(int T, int h, int E) {
  // fp32: chunk partials of the fp32 product; bf16: dL parts, GEMM partials,
  // chunk boundaries and column sums
  const size_t nchunk = size_t(ceil_div(T, kDwTC));
  const size_t f32_ws = al256(nchunk * h * E * 4) + al256(nchunk * E * 4);
  int chunk, nch;
  dwg_chunks(T, h, E, &chunk, &nch);
  const size_t bf_ws = al256(size_t(T) * dwg_e2(E) * 2) + al256(size_t(nch) * h * dwg_e2(E) * 4) +
                       al256(size_t(nch + 1) * 4);
  return al256(size_t(T) * E * 4) + (f32_ws > bf_ws ? f32_ws : bf_ws);
}

size_t router_aux_ws_bytes(int T, int E) { return al256(size_t(ceil_div(T, kAuxTokens)) * E * 4); }

template <bool kF32, bool kYF32>
static void launch_dlogits(const void* dy, const void* yp, const int32_t* dst_row,
                           const int32_t* idx, const float* w, const float* logits,
                           const int32_t* counts, int T, int h, int E, int k, float alpha,
                           float* dL, hipStream_t s) {
  const dim3 grid(ceil_div(T, 4)), block(256);
#define MOE_DL(KM)                                                                               \
  hipLaunchKernelGGL((rbwd_dlogits_kernel<kF32, kYF32, KM>), grid, block, 0, s, dy, yp, dst_row, \
                     idx, w, logits, counts, T, h, E, k, alpha, dL)
  if (k <= 1) MOE_DL(1);
  else if (k <= 2) MOE_DL(2);
  else if (k <= 4) MOE_DL(4);
  else if (k <= 8) MOE_DL(8);
  else MOE_DL(MOE_MAX_TOPK);
#undef MOE_DL
}

int router_bwd(const void* dy, const void* yp, int yp_dtype, const int32_t* dst_row, const int32_t* topk_idx,
               const float* topk_w, const float* logits, const int32_t* counts, int T, int h,
               int E, int k, float alpha, int dtype, const void* x, const void* w_gate,
               const float* dx_in, void* dx, float* dlogits, float* dw_gate, float* dbias,
               void* ws, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const bool f32 = dtype == MOE_F32;
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* dL = dlogits ? dlogits : reinterpret_cast<float*>(w);
  w += al256(size_t(T) * E * 4);

  timer_begin(kTRouterBwd, s);
  const bool yf32 = yp_dtype == MOE_F32;
  if (f32 && yf32)
    launch_dlogits<true, true>(dy, yp, dst_row, topk_idx, topk_w, logits, counts, T, h, E, k, alpha, dL, s);
  else if (f32)
    launch_dlogits<true, false>(dy, yp, dst_row, topk_idx, topk_w, logits, counts, T, h, E, k, alpha, dL, s);
  else if (yf32)
    launch_dlogits<false, true>(dy, yp, dst_row, topk_idx, topk_w, logits, counts, T, h, E, k, alpha, dL, s);
  else
    launch_dlogits<false, false>(dy, yp, dst_row, topk_idx, topk_w, logits, counts, T, h, E, k, alpha, dL, s);
  const size_t n = size_t(h) * E;
  if (f32) {
    const int nchunk = ceil_div(T, kDwTC);
    float* part = reinterpret_cast<float*>(w);
    float* part_b = reinterpret_cast<float*>(w + al256(size_t(nchunk) * h * E * 4));
    const dim3 gdw(h / kDwCols, nchunk);
    hipLaunchKernelGGL(rbwd_dwg_kernel<true>, gdw, dim3(256), 0, s, x, dL, T, h, E, part, part_b);
    hipLaunchKernelGGL(rbwd_dwg_reduce_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s,
                       part, part_b, nchunk, h, E, dw_gate, dbias);
  } else {
    int chunk, nch;
    dwg_chunks(T, h, E, &chunk, &nch);
    const int E2 = dwg_e2(E);
    uint16_t* dlhl = reinterpret_cast<uint16_t*>(w);
    w += al256(size_t(T) * E2 * 2);
    float* P = reinterpret_cast<float*>(w);
    w += al256(size_t(nch) * h * E2 * 4);
    int32_t* choff = reinterpret_cast<int32_t*>(w);
    const size_t nel = size_t(T) * E;
    const int nconv = int(nel / 256 + 1 < 1024 ? nel / 256 + 1 : 1024);
    hipLaunchKernelGGL(rbwd_dl_split_kernel, dim3(unsigned(nconv + (dbias ? E : 0))), dim3(256), 0, s,
                       dL, T, E, E2, chunk, nch, nconv, dlhl, choff, dbias);
    const int rc = dw_rows_bf16(x, h, dlhl, E2, choff, nch, T, P, s);
    if (rc != MOE_OK) {
      timer_end(kTRouterBwd, s);
      return rc;
    }
    hipLaunchKernelGGL(rbwd_dwg_gemm_reduce_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0,
                       s, P, nch, h, E, E2, dw_gate);
  }
  const dim3 gdx(ceil_div(T, kDxTokens), ceil_div(h / 32, kDxCbPer));
  if (f32) {
    hipLaunchKernelGGL(rbwd_dx_kernel<true>, gdx, dim3(256), 0, s, dL, w_gate, dx_in, T, h, E, dx);
  } else if (E <= 64) {
    const uint16_t* wgb = static_cast<const uint16_t*>(w_gate);
    uint16_t* dxb = static_cast<uint16_t*>(dx);
    switch (ceil_div(E, 16)) {
      case 1: hipLaunchKernelGGL(rbwd_dx_bf16_kernel<1>, gdx, dim3(256), 0, s, dL, wgb, dx_in, T, h, E, dxb); break;
      case 2: hipLaunchKernelGGL(rbwd_dx_bf16_kernel<2>, gdx, dim3(256), 0, s, dL, wgb, dx_in, T, h, E, dxb); break;
      case 3: hipLaunchKernelGGL(rbwd_dx_bf16_kernel<3>, gdx, dim3(256), 0, s, dL, wgb, dx_in, T, h, E, dxb); break;
      default: hipLaunchKernelGGL(rbwd_dx_bf16_kernel<4>, gdx, dim3(256), 0, s, dL, wgb, dx_in, T, h, E, dxb); break;
    }
  } else {
    hipLaunchKernelGGL(rbwd_dx_kernel<false>, gdx, dim3(256), 0, s, dL, w_gate, dx_in, T, h, E, dx);
  }
  timer_end(kTRouterBwd, s);
  return launch_status();
}

int router_aux(const float* logits, const int32_t* counts, int T, int E, int k, float alpha,
               float* loss, void* ws, hipStream_t s) {
  float* colsum = static_cast<float*>(ws);
  const int nblk = ceil_div(T, kAuxTokens);
  timer_begin(kTRouterAux, s);
  if (nblk > 0)
    hipLaunchKernelGGL(aux_colsum_kernel, dim3(nblk), dim3(256), size_t(kAuxTokens) * E * 4, s,
                       logits, T, E, colsum);
  hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(256), 0, s, colsum, nblk, counts, T, E, k,
                     alpha, loss);
  timer_end(kTRouterAux, s);
  return launch_status();
}

}  // namespace moe_launch
