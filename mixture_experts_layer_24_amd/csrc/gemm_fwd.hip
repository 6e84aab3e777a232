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
//     four waves of 128 x 128 (4 x 4 MFMA 32x32 blocks, 256 fp32 accumulators
//     per lane, held in AGPRs).  Two LDS stages (128 KB) give one barrier per
//     K step.  Operands go global -> LDS directly (buffer_load ... lds, no
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
#include "common.h"

namespace moe {

constexpr int kBM = 256, kBN = 256, kRowB = 128;  // tile rows, cols, bytes of K per LDS row
constexpr int kStageB = kBM * kRowB;              // bytes of one operand stage (32 KB)
constexpr int kGemmLds = 4 * kStageB;             // A and B, two stages each (128 KB)

enum { kModeFC1 = 0, kModeFC2 = 1 };

struct GemmArgs {
  const void* A;          // [rows][K]
  const float* a_scale;   // FP8: [rows]
  const void* B;          // [E][N][K]
  const float* b_scale;   // FP8: [E][N]
  const int32_t* offsets; // [E+1]
  int E, K, N, rows;
  void* out;              // FC1: act [rows][N/2]; FC2: yp [rows][N]
  void* save;             // FC1: G|U [rows][N] bf16, or null
  uint32_t* row_amax;     // FC1 with FP8: [rows] (fp32 bits, atomic max)
};

__device__ __forceinline__ int lds_pos(int row, int c) {
  return row * kRowB + ((c ^ ((row >> 1) & 7)) << 4);
}

template <int DT>
struct Elem;
template <> struct Elem<MOE_F32> { static constexpr int bytes = 4; };
template <> struct Elem<MOE_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<MOE_FP8_E4M3> { static constexpr int bytes = 1; };

// One 32x32 output block += A-fragment x B-fragment over 32 (bf16, f32) or
// 64 (fp8) bytes of K per row.  The K order inside a fragment pair is the
// same for A and B, which is all a dot product needs.
template <int DT>
struct Frag;
template <> struct Frag<MOE_BF16> {
  u32x4 v;
  static constexpr int kSub = 4;  // substeps per 128-byte LDS row
  static constexpr int kReads = 1, kMfma = 1;  // LDS reads per fragment, MFMAs per pair
  __device__ __forceinline__ void load(const unsigned char* base, int row, int s, int half) {
    v = *reinterpret_cast<const u32x4*>(base + lds_pos(row, 2 * s + half));
  }
  __device__ __forceinline__ static void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
  }
};
template <> struct Frag<MOE_F32> {
  u32x4 v;
  static constexpr int kSub = 4;
  static constexpr int kReads = 1, kMfma = 4;
  __device__ __forceinline__ void load(const unsigned char* base, int row, int s, int half) {
    v = *reinterpret_cast<const u32x4*>(base + lds_pos(row, 2 * s + half));
  }
  __device__ __forceinline__ static void mma(f32x16& c, const Frag& a, const Frag& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v[i]), __uint_as_float(b.v[i]),
                                               c, 0, 0, 0);
  }
};
template <> struct Frag<MOE_FP8_E4M3> {
  u32x4 v0, v1;
  static constexpr int kSub = 2;
  static constexpr int kReads = 2, kMfma = 1;
  __device__ __forceinline__ void load(const unsigned char* base, int row, int s, int half) {
    v0 = *reinterpret_cast<const u32x4*>(base + lds_pos(row, 4 * s + 2 * half));
    v1 = *reinterpret_cast<const u32x4*>(base + lds_pos(row, 4 * s + 2 * half + 1));
  }
  __device__ __forceinline__ static void mma(f32x16& c, const Frag& a, const Frag& b) {
    i32x8 av = {int(a.v0[0]), int(a.v0[1]), int(a.v0[2]), int(a.v0[3]),
                int(a.v1[0]), int(a.v1[1]), int(a.v1[2]), int(a.v1[3])};
    i32x8 bv = {int(b.v0[0]), int(b.v0[1]), int(b.v0[2]), int(b.v0[3]),
                int(b.v1[0]), int(b.v1[1]), int(b.v1[2]), int(b.v1[3])};
    // formats 0/0 = E4M3 x E4M3; E8M0 scales of 127 = 1.0
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
  }
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

struct Tile {
  int e, row0, row_end, n0;
};

// Which expert / m-tile / n-tile the t-th tile is: experts in order, m-tiles
// fastest within an expert, so consecutive tiles share a weight column block.
__device__ __forceinline__ Tile tile_of(int t, const int* tpre, const int* offs, int E) {
  int lo = 0, hi = E - 1;  // expert e with tpre[e] <= t < tpre[e+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tpre[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int mt_e = ceil_div(offs[lo + 1] - offs[lo], kBM);
  const int local = t - tpre[lo];
  const int nt = local / mt_e, mt = local - nt * mt_e;
  return Tile{lo, offs[lo] + mt * kBM, offs[lo + 1], nt * kBN};
}

// Buffer descriptors of a tile's A rows and B rows: reads past the end of
// the A or B array return zero (ragged M tail of the last expert, N tail).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t off, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(static_cast<const unsigned char*>(base) + off), (short)0,
      int(bytes < 0x7FFFFFF0u ? bytes : 0x7FFFFFF0u), 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_ptr_t;

// One K slab (128 bytes per row) of A and B straight from memory into LDS
// stage `st`.  Wave w fills row groups 8w..8w+7 of each operand; within an
// 8-row group lane l lands at LDS byte 16*l (row l/8, position l%8), so it
// fetches the chunk that the XOR swizzle keeps at that position.
__device__ __forceinline__ void issue_slab(unsigned char* lds, int st, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, int wave, int voff_e,
                                           int voff_o, int rowB, int koff) {
  unsigned char* A = lds + st * (2 * kStageB) + wave * 8 * 1024;
  unsigned char* B = A + kStageB;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int v = ((i & 1) ? voff_o : voff_e) + i * 8 * rowB + koff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t*)(A + i * 1024), 16, v, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t*)(B + i * 1024), 16, v, 0, 0, 0);
  }
}

// Fragments of substep s of one LDS stage (4 A and 4 B fragments per wave).
template <int DT>
__device__ __forceinline__ void load_frags(Frag<DT> (&fa)[4], Frag<DT> (&fb)[4],
                                           const unsigned char* As, int arow, int brow, int s,
                                           int half) {
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i].load(As, arow + i * 32, s, half);
#pragma unroll
  for (int j = 0; j < 4; ++j) fb[j].load(As + kStageB, brow + j * 32, s, half);
}

template <int DT>
__device__ __forceinline__ void mma_all(f32x16 (&acc)[4][4], const Frag<DT> (&fa)[4],
                                        const Frag<DT> (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) Frag<DT>::mma(acc[i][j], fa[i], fb[j]);
}

template <int DT, int MODE>
__device__ __forceinline__ void epilogue(const GemmArgs& g, f32x16 (&acc)[4][4], int e, int row0,
                                         int row_end, int n0, int wm, int wn, int half, int l32) {
  const int rbase = row0 + wm * 128;
  if (MODE == kModeFC1) {
    const int hf = g.N / 2;
    const int chb = (n0 + wn * 128) / 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float rmax[16];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int ch = chb + p * 32 + l32;
        const int colg = n0 + wn * 128 + (2 * p) * 32 + l32;  // packed column of G
        float sg = 1.f, su = 1.f;
        if (DT == MOE_FP8_E4M3) {
          sg = g.b_scale[size_t(e) * g.N + colg];
          su = g.b_scale[size_t(e) * g.N + colg + 32];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          float G = acc[i][2 * p][r], U = acc[i][2 * p + 1][r];
          if (DT == MOE_FP8_E4M3) {
            const float xs = row < row_end ? g.a_scale[row] : 0.f;
            G *= xs * sg;
            U *= xs * su;
          }
          const float a = silu_f(G) * U;
          if (row < row_end) {
            if (DT == MOE_BF16) {
              static_cast<uint16_t*>(g.out)[size_t(row) * hf + ch] = uint16_t(f32_to_bf16_bits(a));
            } else {
              // fp32 A; for FP8 the per-row quantization reads this exact value
              static_cast<float*>(g.out)[size_t(row) * hf + ch] = a;
              if (DT == MOE_FP8_E4M3) rmax[r] = p == 0 ? fabsf(a) : fmaxf(rmax[r], fabsf(a));
            }
            if (g.save) {
              uint16_t* sv = static_cast<uint16_t*>(g.save) + size_t(row) * g.N + colg;
              sv[0] = uint16_t(f32_to_bf16_bits(G));
              sv[32] = uint16_t(f32_to_bf16_bits(U));
            }
          } else if (DT == MOE_FP8_E4M3) {
            rmax[r] = 0.f;
          }
        }
      }
      if (DT == MOE_FP8_E4M3) {
        // row max over this wave's 64 channels: reduce over the 32 lanes of a half
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float m = rmax[r];
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          const int row = rbase + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (l32 == 0 && row < row_end) atomicMax(g.row_amax + row, __float_as_uint(m));
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 128 + j * 32 + l32;
        if (col >= g.N) continue;
        float cs = 1.f;
        if (DT == MOE_FP8_E4M3) cs = g.b_scale[size_t(e) * g.N + col];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < row_end) {
            float y = acc[i][j][r];
            if (DT == MOE_FP8_E4M3) y *= g.a_scale[row] * cs;
            if (DT == MOE_F32)
              static_cast<float*>(g.out)[size_t(row) * g.N + col] = y;
            else
              static_cast<uint16_t*>(g.out)[size_t(row) * g.N + col] = uint16_t(f32_to_bf16_bits(y));
          }
        }
      }
  }
}

template <int DT, int MODE>
__global__ void __launch_bounds__(256, 1) grouped_gemm_kernel(GemmArgs g) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int tpre[MOE_MAX_EXPERTS + 1];
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  constexpr int EB = Elem<DT>::bytes;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int NT = ceil_div(g.N, kBN);  // FC2 may end in a 128-column tail

  for (int e = tid; e <= g.E; e += 256) {
    int o = g.offsets[e];
    offs[e] = o < 0 ? 0 : (o > g.rows ? g.rows : o);  // never address past `rows`
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    tpre[0] = 0;
    for (int e = 0; e < g.E; ++e) {
      if (offs[e + 1] < offs[e]) offs[e + 1] = offs[e];
      run += ceil_div(offs[e + 1] - offs[e], kBM) * NT;
      tpre[e + 1] = run;
    }
  }
  __syncthreads();
  const int total = tpre[g.E];
  const int G = gridDim.x;
  const int b = blockIdx.x;
  // the 32 workgroups of one XCD (b % 8) take consecutive tiles
  int t = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  if (t >= total) return;

  const int rowB = g.K * EB;  // bytes per operand row (K * element size)
  const int nk = rowB / kRowB;
  // loader geometry (see issue_slab)
  const int lrow = wave * 64 + (lane >> 3);
  const int sw = (lrow >> 1) & 7;
  const int voff_e = lrow * rowB + (((lane & 7) ^ sw) << 4);
  const int voff_o = lrow * rowB + (((lane & 7) ^ sw ^ 4) << 4);
  // fragment rows inside a stage
  const int arow = wm * 128 + l32, brow = wn * 128 + l32;

  auto rsrc_a = [&](const Tile& c) {
    return rsrc(g.A, size_t(c.row0) * rowB, size_t(g.rows - c.row0) * rowB);
  };
  auto rsrc_b = [&](const Tile& c) {
    return rsrc(g.B, (size_t(c.e) * g.N + c.n0) * rowB, size_t(g.N - c.n0) * rowB);
  };

  constexpr int S = Frag<DT>::kSub;             // substeps per slab (even)
  constexpr int NR = 8 * Frag<DT>::kReads;      // LDS reads per substep
  constexpr int NM = 16 * Frag<DT>::kMfma;      // MFMAs per substep

  Tile cur = tile_of(t, tpre, offs, g.E);
  __amdgpu_buffer_rsrc_t ra = rsrc_a(cur), rb = rsrc_b(cur);
  int st = 0;
  issue_slab(lds, st, ra, rb, wave, voff_e, voff_o, rowB, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  Frag<DT> fa[2][4], fb[2][4];
  load_frags<DT>(fa[0], fb[0], lds, arow, brow, 0, half);

  while (true) {
    const int tn = t + G;
    const bool has_next = tn < total;
    const Tile nxt = has_next ? tile_of(tn, tpre, offs, g.E) : cur;
    const __amdgpu_buffer_rsrc_t ra_n = rsrc_a(nxt), rb_n = rsrc_b(nxt);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int kt = 0; kt < nk; ++kt) {
      // Stage st holds slab kt and fa[0]/fb[0] its first fragments.  Load
      // slab kt+1 (or the next tile's first) into the other stage.
      const bool last = kt + 1 == nk;
      issue_slab(lds, st ^ 1, last ? ra_n : ra, last ? rb_n : rb, wave, voff_e, voff_o, rowB,
                 last ? 0 : (kt + 1) * kRowB);
      const unsigned char* As = lds + st * (2 * kStageB);
#pragma unroll
      for (int s = 0; s + 1 < S; ++s) {
        load_frags<DT>(fa[(s + 1) & 1], fb[(s + 1) & 1], As, arow, brow, s + 1, half);
        mma_all<DT>(acc, fa[s & 1], fb[s & 1]);
      }
      // interleave: one LDS read (and one global load early on) per MFMA
#pragma unroll
      for (int s = 0; s + 1 < S; ++s)
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (s == 0 && q < 16) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      __builtin_amdgcn_s_waitcnt(0);  // stage st read out; slab kt+1 landed
      __syncthreads();
      // next slab's first fragments load while the last substep multiplies
      load_frags<DT>(fa[0], fb[0], lds + (st ^ 1) * (2 * kStageB), arow, brow, 0, half);
      mma_all<DT>(acc, fa[1], fb[1]);
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      st ^= 1;
    }

    epilogue<DT, MODE>(g, acc, cur.e, cur.row0, cur.row_end, cur.n0, wm, wn, half, l32);
    if (!has_next) break;
    t = tn;
    cur = nxt;
    ra = ra_n;
    rb = rb_n;
  }
}

// FP8: act (fp32) -> E4M3 codes with per-row scale amax/448, amax from FC1.
__global__ void __launch_bounds__(256) quant_act_kernel(const float* __restrict__ act,
                                                        const uint32_t* __restrict__ row_amax,
                                                        const int32_t* __restrict__ offsets,
                                                        int E, int hf, uint8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= offsets[E]) return;
  const float amax = __uint_as_float(row_amax[row]);
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (lane == 0) scale[row] = s;
  const f32x4* src = reinterpret_cast<const f32x4*>(act + size_t(row) * hf);
  uint32_t* dst = reinterpret_cast<uint32_t*>(q + size_t(row) * hf);
  for (int c = lane; c < hf / 4; c += 64) {
    f32x4 v = src[c];
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= f32_to_e4m3(v[i] / s) << (8 * i);
    dst[c] = w;
  }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace moe

namespace moe_launch {
using namespace moe;

static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

size_t grouped_fwd_ws_bytes(int rows, int h, int h_ffn, int E, int dtype) {
  (void)h; (void)E;
  size_t r = size_t(rows), hf = size_t(h_ffn);
  size_t act = al256(r * hf * (dtype == MOE_BF16 ? 2 : 4));
  if (dtype == MOE_FP8_E4M3) act += al256(r * hf) + 2 * al256(r * 4);
  return act;
}

template <int DT, int MODE>
static int launch_gemm(const GemmArgs& a, hipStream_t s) {
  static bool attr = allow_lds(grouped_gemm_kernel<DT, MODE>, kGemmLds);
  if (!attr) return MOE_ERR_HIP;
  // upper bound of the tile count, known without reading offsets
  long mt_max = (long(a.rows) + kBM - 1) / kBM + a.E;
  long tiles = mt_max * ((a.N + kBN - 1) / kBN);
  int grid = num_cus();
  if (tiles < grid) grid = int(tiles);
  if (grid < 1) grid = 1;
  timer_begin(MODE == kModeFC1 ? kTFc1 : kTFc2, s);
  hipLaunchKernelGGL((grouped_gemm_kernel<DT, MODE>), dim3(grid), dim3(256), kGemmLds, s, a);
  timer_end(MODE == kModeFC1 ? kTFc1 : kTFc2, s);
  return launch_status();
}

template <int DT>
static int fwd_typed(const void* xp, const float* xp_scale, const moe_weights* W,
                     const int32_t* offsets, int rows, void* h13_save, void* yp, void* ws,
                     hipStream_t s) {
  const int h = W->h, hf = W->h_ffn, E = W->E;
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* act = w;
  size_t act_b = al256(size_t(rows) * hf * (DT == MOE_BF16 ? 2 : 4));
  uint8_t* actq = nullptr;
  uint32_t* amax = nullptr;
  float* ascale = nullptr;
  if (DT == MOE_FP8_E4M3) {
    actq = reinterpret_cast<uint8_t*>(w + act_b);
    amax = reinterpret_cast<uint32_t*>(w + act_b + al256(size_t(rows) * hf));
    ascale = reinterpret_cast<float*>(w + act_b + al256(size_t(rows) * hf) + al256(size_t(rows) * 4));
    hipLaunchKernelGGL(fill_u32_kernel, dim3(ceil_div(rows, 256)), dim3(256), 0, s, amax,
                       size_t(rows), 0u);
  }
  GemmArgs a1{xp, xp_scale, W->w13, W->w13_scale, offsets, E, h, 2 * hf, rows,
              act, h13_save, amax};
  int rc = launch_gemm<DT, kModeFC1>(a1, s);
  if (rc) return rc;
  if (DT == MOE_FP8_E4M3) {
    timer_begin(kTQuant, s);
    hipLaunchKernelGGL(quant_act_kernel, dim3(ceil_div(rows, 4)), dim3(256), 0, s,
                       (const float*)act, amax, offsets, E, hf, actq, ascale);
    timer_end(kTQuant, s);
    GemmArgs a2{actq, ascale, W->w2, W->w2_scale, offsets, E, hf, h, rows, yp, nullptr, nullptr};
    return launch_gemm<DT, kModeFC2>(a2, s);
  }
  GemmArgs a2{act, nullptr, W->w2, nullptr, offsets, E, hf, h, rows, yp, nullptr, nullptr};
  return launch_gemm<DT, kModeFC2>(a2, s);
}

int grouped_fwd(const void* xp, const float* xp_scale, const moe_weights* W,
                const int32_t* offsets, int rows, void* h13_save, void* yp, void* ws,
                hipStream_t s) {
  if (rows == 0) return MOE_OK;
  switch (W->dtype) {
    case MOE_F32: return fwd_typed<MOE_F32>(xp, xp_scale, W, offsets, rows, h13_save, yp, ws, s);
    case MOE_BF16: return fwd_typed<MOE_BF16>(xp, xp_scale, W, offsets, rows, h13_save, yp, ws, s);
    case MOE_FP8_E4M3:
      return fwd_typed<MOE_FP8_E4M3>(xp, xp_scale, W, offsets, rows, h13_save, yp, ws, s);
  }
  return MOE_ERR_DTYPE;
}

}  // namespace moe_launch
