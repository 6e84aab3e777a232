// Router: gate GEMM + top-k + softmax over the selected logits.
//
// Gate scores and top-k selection: MegaScale-MoE paper review, §三 (MoE
// layer structure, Fig. 2; training flow "token routing"); DisagMoE page,
// §2.1 / Fig. 2(a) (k highest-scoring experts, weighted sum).  Softmax over
// the k kept logits and the tie rule (lower expert index first) are this
// library's reading of the unspecified details.
//
// BF16: logits on MFMA with x read once from HBM: for E a multiple of 8 up
// to 64, route_tr_kernel (W_g rows as loaded, fragments through the LDS
// transpose read); other E, route_bf16_kernel (W_g transposed through LDS).
// FP32 (small workloads) and given logits: a plain dot-product kernel.  Top-k
// runs on eight lanes per token.
#include "common.h"

namespace moe {

constexpr int kRouteTokens = 128;  // tokens per workgroup of the generic kernel

// Top-k of one token's E logits and the softmax over the k kept ones, by 8
// cooperating lanes (lanes 8q .. 8q+7 of a wave, `sub` = lane % 8).  Slot j
// holds the j-th expert in the order (logit descending, expert index
// ascending), so equal logits keep the lower index first.  Lane sub holds
// experts sub, sub + 8, ... in registers (ME8 >= ceil(E / 8) of them); round j
// takes every lane's best expert not yet taken and reduces the eight
// candidates by shuffles.  Lane sub = 0 writes the k ids and weights.
template <int ME8>
__device__ __forceinline__ void topk_select8(const float* L, int E, int k, int sub,
                                             int32_t* idx_out, float* w_out) {
  static_assert(ME8 <= 32, "taken mask");
  float v[ME8];
  uint32_t taken = 0;
#pragma unroll
  for (int m = 0; m < ME8; ++m) {
    const int e = sub + 8 * m;
    v[m] = e < E ? L[e] : 0.f;
    if (e >= E) taken |= 1u << m;
  }
  float vals[MOE_MAX_TOPK];
  int ids[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int be = -1;
#pragma unroll
    for (int m = 0; m < ME8; ++m) {
      const int e = sub + 8 * m;
      if (!((taken >> m) & 1u) && (be < 0 || v[m] > bv)) { bv = v[m]; be = e; }
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      const float ov = __shfl_xor(bv, off, 8);
      const int oe = __shfl_xor(be, off, 8);
      if (oe >= 0 && (be < 0 || ov > bv || (ov == bv && oe < be))) { bv = ov; be = oe; }
    }
    vals[j] = bv;
    ids[j] = be;
    if (be >= 0 && (be & 7) == sub) taken |= 1u << (be >> 3);
  }
  if (sub != 0) return;
  float z[MOE_MAX_TOPK];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j >= k) break;
    z[j] = expf(vals[j] - vals[0]);
    sum += z[j];
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j >= k) break;
    idx_out[j] = ids[j];
    w_out[j] = (k == 1) ? 1.0f : z[j] * inv;
  }
}

// BF16 logits on MFMA 32x32x16: one workgroup of four (or eight, see RES)
// waves per 32 tokens; wave w takes the K range [w h/NW, (w+1) h/NW) in
// 64-element chunks.
// x goes straight from HBM into A fragments (64 contiguous bytes per lane
// per chunk), one chunk (three with W_g resident) ahead of its MFMAs.  The chunk's 64 rows of W_g are
// one contiguous block: the wave reads it in 16-byte loads (lane = row, up to
// eight loads of a lane issued together) and writes it transposed into its
// own LDS region ([expert][k], 144-byte rows), from where each lane's B
// fragment is one 16-byte read.  The waves' partial 32 x E tiles are summed in LDS in wave
// order, the bias added, and eight lanes per token pick its k experts.
constexpr int kRtTokens = 32;
constexpr int kRtChunk = 64;                // K elements per chunk
constexpr int kRtStride = kRtChunk + 8;     // bf16 per LDS row of W^T

// RES: eight waves (two per SIMD) split h, and each wave's whole K range of
// W_g (E x h/8 values) is staged in LDS once, transposed ([E][h/8 + 8]), when
// all eight ranges fit; the chunk loop then runs without barriers or W_g
// loads.  Otherwise four waves split h and stage W_g chunk by chunk.
template <int NT, bool RES>  // NT = ceil(E / 32) expert blocks of 32
__global__ void __launch_bounds__(RES ? 512 : 256) route_bf16_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wg,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits_out, int T,
                                                         int h, int E, int k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int t0 = blockIdx.x * kRtTokens;
  const int row = t0 + l32;
  const int rowc = row < T ? row : T - 1;
  constexpr int NW = RES ? 8 : 4;  // waves
  const int kw = h / NW;  // h is a multiple of 64 (of 128 with RES), so kw of 16
  // K ranges rotated by workgroup (see route_tr_kernel); partial tiles are
  // summed in range order
  const int kr = (wave + int(blockIdx.x)) % NW;
  const int kbeg = kr * kw;
  // this wave's W^T region: [NT*32][kRtStride] bf16 per chunk, or (RES) the
  // whole range [E][kw + 8]
  const int rstride = RES ? kw + 8 : kRtStride;
  uint16_t* wt = reinterpret_cast<uint16_t*>(smem) +
                 size_t(wave) * (RES ? size_t(E) * rstride : size_t(NT) * 32 * kRtStride);
  if (RES) {
    // lane = row kk of the range, 16-byte units of 8 experts (E % 8 == 0),
    // else single values; eight loads in flight per lane
    const uint16_t* src = wg + size_t(kbeg) * E;
    if ((E & 7) == 0) {
      const int ne8 = E / 8, nu = kw * ne8;
      for (int u0 = lane; u0 < nu; u0 += 64 * 8) {
        u32x4 v[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int u = u0 + 64 * b;
          if (u < nu) v[b] = *reinterpret_cast<const u32x4*>(src + size_t(u % kw) * E + (u / kw) * 8);
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int u = u0 + 64 * b;
          if (u >= nu) break;
          const int kk = u % kw, e8 = u / kw;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            wt[(e8 * 8 + i) * rstride + kk] = uint16_t(v[b][i >> 1] >> (16 * (i & 1)));
        }
      }
    } else {
      for (int q = lane; q < kw * E; q += 64) {
        const int kk = q / E, e = q - kk * E;
        wt[e * rstride + kk] = src[q];
      }
    }
    __syncthreads();
  }

  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;

  const uint16_t* xr = x + size_t(rowc) * h + half * 32;
  // x fragments of chunk kc (zero past the wave's K range)
  auto load_x = [&](int kc, u32x4 (&xa)[4]) {
    const int kn = kbeg + kw - kc < kRtChunk ? kbeg + kw - kc : kRtChunk;  // <= 0: none
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xa[s] = (half * 32 + s * 8 < kn) ? *reinterpret_cast<const u32x4*>(xr + kc + s * 8)
                                       : u32x4{0, 0, 0, 0};
  };
  constexpr int kWB = 8;  // W_g units (8 experts) per lane loaded before their LDS stores
  // x runs PF chunks ahead of the MFMAs (RES: three, with no barrier in the
  // loop to pace the waves; else one, during the W_g staging)
  constexpr int PF = RES ? 3 : 1;
  u32x4 xq[PF + 1][4];
#pragma unroll
  for (int p = 0; p < PF; ++p) load_x(kbeg + p * kRtChunk, xq[p]);
  for (int kc = kbeg; kc < kbeg + kw; kc += kRtChunk) {
    const int kn = kbeg + kw - kc < kRtChunk ? kbeg + kw - kc : kRtChunk;  // 16, 32, 48 or 64
    load_x(kc + PF * kRtChunk, xq[PF]);
    u32x4 (&xa)[4] = xq[0];
    // W_g rows kc .. kc+kn-1 are kn*E contiguous values.  With E % 8 == 0,
    // lane kk takes row kc + kk in 16-byte units of 8 experts (the first kWB
    // units loaded before the barrier) and stores them transposed, so
    // neighbouring lanes store neighbouring k of one expert row of W^T;
    // otherwise the units run in memory order.
    const uint16_t* src = wg + size_t(kc) * E;
    if (RES) {
      // W^T of the whole range is resident
    } else if ((E & 7) == 0) {
      const int ne8 = E / 8;
      const bool rowok = lane < kn;
      u32x4 wv[kWB];
#pragma unroll
      for (int b = 0; b < kWB; ++b)
        if (rowok && b < ne8) wv[b] = *reinterpret_cast<const u32x4*>(src + size_t(lane) * E + b * 8);
      __syncthreads();  // previous chunk's fragments read out of wt
      for (int e0 = 0; e0 < ne8; e0 += kWB) {
        if (e0 > 0) {
#pragma unroll
          for (int b = 0; b < kWB; ++b)
            if (rowok && e0 + b < ne8)
              wv[b] = *reinterpret_cast<const u32x4*>(src + size_t(lane) * E + (e0 + b) * 8);
        }
#pragma unroll
        for (int b = 0; b < kWB; ++b) {
          if (!rowok || e0 + b >= ne8) continue;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            wt[((e0 + b) * 8 + i) * kRtStride + lane] = uint16_t(wv[b][i >> 1] >> (16 * (i & 1)));
        }
      }
    } else {
      __syncthreads();  // previous chunk's fragments read out of wt
      const int units = kn * E / 8;
      for (int u = lane; u < units; u += 64) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + size_t(u) * 8);
        int q = u * 8, kk = q / E, e = q - kk * E;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          wt[e * kRtStride + kk] = uint16_t(v[i >> 1] >> (16 * (i & 1)));
          if (++e == E) { e = 0; ++kk; }
        }
      }
    }
    if (!RES) __syncthreads();
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = n * 32 + l32;
      const uint16_t* br = RES ? wt + e * rstride + (kc - kbeg) + half * 32 : wt + e * kRtStride + half * 32;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 b = (e < E && half * 32 + s * 8 < kn) ? *reinterpret_cast<const u32x4*>(br + s * 8)
                                                   : u32x4{0, 0, 0, 0};
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, xa[s]), __builtin_bit_cast(bf16x8, b), acc[n], 0, 0, 0);
      }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
      for (int s = 0; s < 4; ++s) xq[p][s] = xq[p + 1][s];
  }
  __syncthreads();
  // partial tiles -> LDS [K range][token][E], then sum in range order
  float* part = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int e = n * 32 + l32;
    if (e < E) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * half + (r & 3);
        part[(kr * kRtTokens + i) * E + e] = acc[n][r];
      }
    }
  }
  __syncthreads();
  // the sum replaces wave 0's partial in place: logits [32][E]
  for (int q = tid; q < kRtTokens * E; q += NW * 64) {
    float v = part[q];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += part[w * kRtTokens * E + q];
    const int i = q / E, e = q - i * E;
    if (bias) v += bias[e];
    part[q] = v;
    if (logits_out && t0 + i < T) logits_out[size_t(t0) * E + q] = v;
  }
  __syncthreads();
  // eight lanes per token (256 threads = 32 tokens)
  {
    const int i = tid >> 3, t = t0 + i;
    if (i < kRtTokens && t < T)
      topk_select8<4 * NT>(part + i * E, E, k, tid & 7, topk_idx + size_t(t) * k,
                           topk_w + size_t(t) * k);
  }
}

// BF16 logits with W_g read in its own [h][E] layout (E a multiple of 8, at
// most 64): eight waves (E = 8: sixteen; E >= 32: four) share out h in
// 64-row chunks.  x goes from HBM straight into A fragments (64 contiguous bytes per lane per
// chunk); the chunk's W_g rows come into registers with 16-byte loads and
// are written unchanged into the wave's own LDS buffer, from where transpose
// reads (ds_read_b64_tr_b16) hand each lane four K-consecutive values of one
// expert column: W_g is never rearranged.  x runs three chunks ahead of the
// MFMAs, W_g three (E > 32: two); the waves meet only to sum their partial
// 32 x E tiles (in wave order), add the bias and pick the top k.
typedef __attribute__((address_space(3))) void rt_lds_t;
typedef short rt_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) rt_s16x4 rt_lds_s16x4;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rt_rsrc(const void* base, size_t off, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(static_cast<const unsigned char*>(base) + off), (short)0,
      int(bytes < 0x7FFFFFF0u ? bytes : 0x7FFFFFF0u), 0x00020000);
}

template <int E8, int NW>  // E = 8 E8; NW waves split h
__global__ void __launch_bounds__(NW * 64) route_tr_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wg,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ logits_out, int T,
                                                           int h, int E, int k,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w) {
  static_assert(E8 >= 1 && E8 <= 8, "E <= 64");
  constexpr int NT = (E8 + 3) / 4;  // 32-expert blocks
  constexpr int RB = 16 * E8;       // bytes per W_g row
  constexpr int CB = 64 * RB;       // bytes per 64-row chunk: E8 pieces of 1 KB
  // W_g chunks in flight: four register slots (loaded three chunks ahead), or
  // for E > 32 two (two ahead), which keeps a wave within its registers
  constexpr int WS = E8 <= 4 ? 4 : 2, WD = WS == 4 ? 3 : 2;
  // 128-byte rows: rows 2 and 3 (mod 4) keep their 16-byte pieces at p ^ 4,
  // so the four rows of a transpose read fall on distinct banks
  constexpr bool kSwz = E8 == 8;
  constexpr int NQ = (kRtTokens * 8 * E8 + NW * 64 - 1) / (NW * 64);  // logits summed per thread
  // a wave's chunk buffer; after the K loop the partial tiles [NW][32][E] fp32
  __shared__ __align__(16) unsigned char wbuf[NW * CB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int t0 = blockIdx.x * kRtTokens;
  // The 64-row K chunks are dealt to the waves in turn (wave w: chunks w,
  // w + NW, ...), so at any time the workgroup's waves read one contiguous
  // span of every row (DRAM pages are opened for long runs, not 128 bytes
  // per row), and each workgroup starts at its own place in its waves'
  // sequences (with all of them at the same row offsets at once, a
  // power-of-two row pitch would put their reads on a few HBM channels).
  // A wave's partial tile is its chunks' products summed in its own order;
  // the tiles are summed in wave order.
  const int ncht = h / 64;                     // chunks of a row
  const int nch = (ncht + NW - 1) / NW;        // steps per wave (chunks past ncht read zero)
  const int rot = int(blockIdx.x) % nch;
  auto chunk = [&](int j) { return (j + rot < nch ? j + rot : j + rot - nch) * NW + wave; };
  const int nrow = T - t0 < kRtTokens ? T - t0 : kRtTokens;
  // x rows t0 .. t0 + nrow - 1 and all of W_g: the buffer descriptors read
  // zero past them
  const __amdgpu_buffer_rsrc_t rx = rt_rsrc(x, size_t(t0) * h * 2, size_t(nrow) * h * 2);
  const __amdgpu_buffer_rsrc_t rw = rt_rsrc(wg, 0, size_t(h) * RB);
  const int xoff = (l32 * h + half * 32) * 2;
  unsigned char* buf = wbuf + wave * CB;
  // where lane l writes its 16 bytes of each 1 KB piece of a chunk
  const int wpos = kSwz ? (lane >> 3) * RB + (((lane & 7) ^ (((lane >> 4) & 1) * 4)) << 4) : lane * 16;
  // transpose-read offsets: lanes 4j .. 4j+3 of a 16-lane group address row j
  // of a 4-row block, columns 4 (lane & 3) + 16 g (+ 32 nb); lane i of the
  // group receives column i.  Columns past E wrap onto real ones: they only
  // feed output columns past E, which are never read.
  int tro[NT];
#pragma unroll
  for (int nb = 0; nb < NT; ++nb) {
    const int r = (lane & 15) >> 2;
    const int byte = ((nb * 32 + ((lane >> 4) & 1) * 16 + 4 * (lane & 3)) % E) * 2;
    const int piece = kSwz ? ((byte >> 4) ^ (((r >> 1) & 1) * 4)) : (byte >> 4);
    tro[nb] = (half * 32 + r) * RB + piece * 16 + (byte & 15);
  }
  // x chunk c sits in register slot c % 4, W_g chunk c in slot c % WS
  u32x4 xq[4][4], wq[WS][E8];
  // (step j works on chunk chunk(j))
  // a chunk past the row's end (h / 64 not a multiple of NW) is loaded from
  // an offset beyond the descriptor, which reads zeros (in place it would
  // read the next row); W_g reads zero there too, so such a chunk adds 0
  auto load_x = [&](int j, u32x4(&xa)[4]) {
    const int g = chunk(j);
    const int so = g < ncht ? g * 128 : (1 << 30);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xa[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff + s * 16, so, 0));
  };
  auto load_w = [&](int j, u32x4(&wa)[E8]) {
    const int g = chunk(j);
#pragma unroll
    for (int i = 0; i < E8; ++i)
      wa[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, lane * 16, g * CB + i * 1024, 0));
  };
  auto put = [&](const u32x4(&wa)[E8]) {
#pragma unroll
    for (int i = 0; i < E8; ++i) *reinterpret_cast<u32x4*>(buf + i * 1024 + wpos) = wa[i];
  };
  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  // the bias of the logits this thread sums at the end
  float bq[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = tid + j * NW * 64;
    bq[j] = bias && q < kRtTokens * E ? bias[q % E] : 0.f;
  }

#pragma unroll
  for (int p = 0; p < 3; ++p)
    if (p < nch) load_x(p, xq[p]);
#pragma unroll
  for (int p = 0; p < WD; ++p)
    if (p < nch) load_w(p, wq[p]);
  put(wq[0]);
  // chunk c (Q = c % 4, known in each copy of the step): load x chunk c + 3
  // and W_g chunk c + WD, multiply chunk c out of the LDS buffer, then write
  // chunk c + 1 into it (a wave's LDS operations run in order, so the reads of
  // chunk c come first)
  auto step = [&](auto qc, int c) {
    constexpr int Q = decltype(qc)::value;
    if (c + 3 < nch) load_x(c + 3, xq[(Q + 3) & 3]);
    if (c + WD < nch) load_w(c + WD, wq[(Q + WD) % WS]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 xa = xq[Q][s];
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) {
        const unsigned char* p = buf + tro[nb] + s * 8 * RB;
        const rt_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((rt_lds_s16x4*)(rt_lds_t*)p);
        const rt_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((rt_lds_s16x4*)(rt_lds_t*)(p + 4 * RB));
        const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
        const u32x4 bf = u32x4{a[0], a[1], b[0], b[1]};
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa),
                                                         __builtin_bit_cast(bf16x8, bf), acc[nb], 0, 0, 0);
      }
    }
    if (c + 1 < nch) put(wq[(Q + 1) % WS]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  int c = 0;
  for (; c + 3 < nch; c += 4) {
    step(I0{}, c);
    step(I1{}, c + 1);
    step(I2{}, c + 2);
    step(I3{}, c + 3);
  }
  if (c < nch) step(I0{}, c);
  if (c + 1 < nch) step(I1{}, c + 1);
  if (c + 2 < nch) step(I2{}, c + 2);
  __syncthreads();
  // partial tiles -> LDS [wave][token][E], then sum in wave order
  float* part = reinterpret_cast<float*>(wbuf);
#pragma unroll
  for (int nb = 0; nb < NT; ++nb) {
    const int e = nb * 32 + l32;
    if (e < E) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * half + (r & 3);
        part[(wave * kRtTokens + i) * E + e] = acc[nb][r];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = tid + j * NW * 64;
    if (q < kRtTokens * E) {
      float v = part[q];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += part[w * kRtTokens * E + q];
      part[q] = v + bq[j];
    }
  }
  __syncthreads();
  {
    const int i = tid >> 3, t = t0 + i;
    if (i < kRtTokens && t < T)
      topk_select8<E8>(part + i * E, E, k, tid & 7, topk_idx + size_t(t) * k, topk_w + size_t(t) * k);
  }
  // the logits last: no barrier waits for these stores
  if (logits_out) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = tid + j * NW * 64;
      if (q < nrow * E) logits_out[size_t(t0) * E + q] = part[q];
    }
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
  // eight lanes per token, 32 tokens per pass
  for (int i = tid >> 3; i < kRouteTokens; i += 32) {
    const int t = t0 + i;
    if (t < T)
      topk_select8<MOE_MAX_EXPERTS / 8>(lg + i * ls, E, k, tid & 7, topk_idx + size_t(t) * k,
                                        topk_w + size_t(t) * k);
  }
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

template <int NT>
static void launch_route_bf16(const void* x, const void* wg, const float* bias, float* logits,
                              int T, int h, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  const dim3 grid(ceil_div(T, kRtTokens));
  // the whole of W_g resident in LDS (eight waves) when it and the eight
  // partial tiles fit in 150 KB
  const size_t resb = size_t(8) * E * (h / 8 + 8) * 2;
  const size_t redb8 = size_t(8) * kRtTokens * E * 4;
  const size_t shm8 = resb > redb8 ? resb : redb8;
  if (h % 128 == 0 && shm8 <= 150 * 1024) {
    static bool ok = allow_lds(route_bf16_kernel<NT, true>, 160 * 1024);
    (void)ok;
    hipLaunchKernelGGL((route_bf16_kernel<NT, true>), grid, dim3(512), shm8, s,
                       (const uint16_t*)x, (const uint16_t*)wg, bias, logits, T, h, E, k, idx, w);
    return;
  }
  const dim3 block(256);
  const size_t redb = size_t(4) * kRtTokens * E * 4;
  const size_t wtb = size_t(4) * NT * 32 * kRtStride * 2;
  static bool ok = allow_lds(route_bf16_kernel<NT, false>, 160 * 1024);
  (void)ok;
  hipLaunchKernelGGL((route_bf16_kernel<NT, false>), grid, block, wtb > redb ? wtb : redb, s,
                     (const uint16_t*)x, (const uint16_t*)wg, bias, logits, T, h, E, k, idx, w);
}

int route(const void* x, const void* w_gate, const float* bias, float* logits, int T, int h,
          int E, int k, int dtype, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (T == 0) return MOE_OK;
  timer_begin(kTRoute, s);
  if (x && dtype == MOE_BF16 && E % 8 == 0 && E <= 64) {
    // sixteen waves (each K range a multiple of 8) where E = 8 keeps a
    // wave's registers within the 128 that four waves per SIMD allow; for
    // E >= 32 four waves, so two workgroups fit a CU (150-170 VGPRs) and each
    // wave walks twice the chunks (DeepSeekMoE-shaped, E = 64: 31.8 -> 25.4
    // us; 352B-shaped, E = 32: 18.1 -> 16.5 us, standalone)
    const bool w16 = h % 128 == 0 && E == 8;
    const dim3 grid(ceil_div(T, kRtTokens)), block(w16 ? 1024 : (E >= 32 ? 256 : 512));
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* wb = (const uint16_t*)w_gate;
    switch (E / 8 + (w16 ? 8 : 0)) {
#define MOE_RT(n, e8, nw)                                                                          \
  case n:                                                                                          \
    hipLaunchKernelGGL((route_tr_kernel<e8, nw>), grid, block, 0, s, xb, wb, bias, logits, T, h,  \
                       E, k, topk_idx, topk_w);                                                    \
    break;
      MOE_RT(1, 1, 8) MOE_RT(2, 2, 8) MOE_RT(3, 3, 8) MOE_RT(4, 4, 4) MOE_RT(5, 5, 4)
      MOE_RT(6, 6, 4) MOE_RT(7, 7, 4) MOE_RT(8, 8, 4) MOE_RT(9, 1, 16)
#undef MOE_RT
    }
  } else if (x && dtype == MOE_BF16) {
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
