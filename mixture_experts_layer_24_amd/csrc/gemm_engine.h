// GroupedGEMM engine shared by the forward and backward passes.
//
// C[m][n] = sum_k A[m][k] * B[n][k] for every expert, both operands
// K-contiguous, fp32 accumulation on MFMA 32x32 (bf16 x16, fp32 x2, fp8 x64).
// Three schedules:
//   SchedM -- rows of A are the expert-contiguous routed rows (ragged M per
//             expert, offsets on device), K fixed: the forward FC1/FC2 and the
//             backward dA / dXp products;
//   SchedK -- every expert has a fixed M x N output and a ragged K = its row
//             count (padded with zeros to whole 128-byte slabs: 128 rows in
//             FP8): the FP8 weight gradients, on transposed operands;
//   SchedKR -- the same products read straight from the row-major routed
//             arrays ([rows][M] and [rows][N], K = the expert's rows): K slabs
//             of 64 rows land in LDS M-major and the fragments come out
//             through the LDS transpose read (BF16 weight gradients).
// Every product runs 256 x 256 tiles on eight waves of 128 x 64 (two per
// SIMD, 128 fp32 accumulators per lane); operands go global -> LDS with
// buffer_load ... lds into two XOR-swizzled stages of 128-byte rows.
#pragma once
#include "common.h"

namespace moe {

// SchedK: per-expert K (rows) padded to one 128-byte slab of the element type
template <int DT>
constexpr int kpad_elems() { return DT == MOE_FP8_E4M3 ? 128 : DT == MOE_F32 ? 32 : 64; }
constexpr int kMaxGrid = 256;  // persistent grid cap (workgroups)
constexpr int kMaxSplit = 8;   // K splits of one tile in the last round

// Tile shape: WM x WN waves, each owning MI x NJ MFMA blocks of 32 x 32, and
// OCC workgroups resident per CU.  The tile is (32 WM MI) x (32 WN NJ).  A K
// slab is ROWB bytes of every A and B row of the tile; LDS holds NS slabs in
// a ring and the loads run NS-1 slabs ahead of the MFMAs.
template <int WM, int WN, int MI, int NJ, int OCC, int ROWB, int NS>
struct GemmCfg {
  static constexpr int kWM = WM, kWN = WN, kMI = MI, kNJ = NJ, kOcc = OCC;
  static constexpr int kRowB = ROWB, kStages = NS;
  static constexpr int kNW = WM * WN;             // waves per workgroup
  static constexpr int kThreads = 64 * kNW;
  static constexpr int kWavesPerSimd = kNW * OCC / 4;
  static constexpr int kBM = 32 * WM * MI, kBN = 32 * WN * NJ;
  static constexpr int kAStage = kBM * ROWB;      // A part of a stage
  static constexpr int kStage = (kBM + kBN) * ROWB;
  static constexpr int kLds = NS * kStage;
  static constexpr int kRowsPerLoad = 1024 / ROWB;  // rows one 1 KB wave load fills
  static constexpr int kGA = kBM / kRowsPerLoad / kNW, kGB = kBN / kRowsPerLoad / kNW;
  static_assert(ROWB == 64 || ROWB == 128, "row pitch");
  static_assert(NS >= 2 && NS <= 4, "stages");
  static_assert(kGA * kRowsPerLoad * kNW == kBM && kGB * kRowsPerLoad * kNW == kBN,
                "rows must split over waves");
  static_assert(kNW % 4 == 0, "whole waves per SIMD");
};

// 256 x 256 on eight waves of 128 x 64 (two per SIMD, so one can issue MFMAs
// while the other waits on a load), 128-byte slabs in two stages (128 KB of
// LDS; one slab in flight while the MFMAs consume the other).  Measured on the
// Mixtral-shaped FC1, this beats four waves of 128 x 128 (whose 256
// accumulators per lane push the epilogue into spills) and 64-byte slabs in
// three or four stages (twice the barriers per K).
template <int DT>
struct CfgFor {
  using type = GemmCfg<2, 4, 4, 2, 1, 128, 2>;
};
template <>
struct CfgFor<MOE_FP8_E4M3> {
  using type = GemmCfg<2, 4, 4, 2, 1, 128, 2>;
};

enum { kSchedM = 0, kSchedK = 1, kSchedKR = 2 };
enum {
  kModeFC1 = 0,   // SiLU(G)*U epilogue (+ optional G|U keep, FP8 row amax)
  kModeFC2 = 1,   // plain output [rows][N] (bf16 / fp32; FP8 rescale)
  kModeBwdDA = 2, // dG, dU from dA and the kept G|U; also A = SiLU(G)*U
  kModeDW = 3,    // fp32 [E][M][N]
  kModeDW13 = 4,  // fp32 [E][M][2*h_ffn packed] split into dW1 / dW3
  kModeFC1Arr = 5,  // FC1 (bf16) whose row tiles wait until a concurrent dispatch copy has
                    // released their rows (see GemmArgs::ready)
};

struct GemmArgs {
  const void* A;          // SchedM: [rows][K]; SchedK: expert e at kpre[e]*M elements, [M][K_e];
                          // SchedKR: [rows][M]
  const float* a_scale;   // FP8: SchedM [rows]; SchedK [E][M]
  const void* B;          // SchedM: [E][N][K]; SchedK: expert e at kpre[e]*N elements, [N][K_e];
                          // SchedKR: [rows][N]
  const float* b_scale;   // FP8: [E][N]
  const int32_t* offsets; // [E+1]
  int E, K, N, rows, M;   // K: SchedM only; M: SchedK / SchedKR only
  void* out;              // see the modes
  void* out2;             // BwdDA: A [rows][N]; DW13: dW3
  void* save;             // FC1: G|U out [rows][N] bf16 or null; BwdDA: G|U in [rows][2N]
  float* row_amax;        // FC1 with FP8: [rows][ceil(N / BN)] row maxima of |A|, one per column tile;
                          // BwdDA with FP8, or null: per expert the column maxima of the stored |A|
                          // ([E][N]), then of |dG|dU| ([E][2N], packed columns), raised by atomic max
                          // from zero
  float* part;            // split-K partial tiles (kMaxGrid tiles) or null: no split
  uint32_t* cnt;          // split-K arrival counters [kMaxGrid], zero before the launch
  int out_f32;            // FC2: 1 stores the output in fp32 (bf16 and FP8 operands too)
  // FC1Arr: rows of each expert that the dispatch copy has written and
  // released, the rows written in all, a word set to 1 if a wait gave up, and
  // the polls after which a wait gives up
  const uint32_t* ready;
  const uint32_t* done;
  int32_t* status;
  int spin_limit;
};

// LDS byte position of 16-byte chunk c of row r (pitch RB bytes): chunks are
// XOR-swizzled by (r / (256/RB)) % (RB/16), so the rows that one 256-byte
// bank sweep covers use every chunk position once and the 64 lanes of a
// fragment read hit distinct banks.
template <int RB>
__device__ __forceinline__ int lds_pos(int row, int c) {
  return row * RB + ((c ^ ((row / (256 / RB)) % (RB / 16))) << 4);
}

template <int DT>
struct Elem;
template <> struct Elem<MOE_F32> { static constexpr int bytes = 4; };
template <> struct Elem<MOE_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<MOE_FP8_E4M3> { static constexpr int bytes = 1; };

// One 32x32 output block += A-fragment x B-fragment over kKBytes of K per
// row (16 bf16, 8 fp32 or 64 fp8 values).  The K order inside a fragment
// pair is the same for A and B, which is all a dot product needs.
template <int DT>
struct Frag;
template <> struct Frag<MOE_BF16> {
  u32x4 v;
  static constexpr int kKBytes = 32;
  static constexpr int kReads = 1, kMfma = 1;  // LDS reads per fragment, MFMAs per pair
  template <int RB>
  __device__ __forceinline__ void load(const unsigned char* base, int row, int s, int half) {
    v = *reinterpret_cast<const u32x4*>(base + lds_pos<RB>(row, 2 * s + half));
  }
  __device__ __forceinline__ static void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
  }
};
template <> struct Frag<MOE_F32> {
  u32x4 v;
  static constexpr int kKBytes = 32;
  static constexpr int kReads = 1, kMfma = 4;
  template <int RB>
  __device__ __forceinline__ void load(const unsigned char* base, int row, int s, int half) {
    v = *reinterpret_cast<const u32x4*>(base + lds_pos<RB>(row, 2 * s + half));
  }
  __device__ __forceinline__ static void mma(f32x16& c, const Frag& a, const Frag& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v[i]), __uint_as_float(b.v[i]),
                                               c, 0, 0, 0);
  }
};
template <> struct Frag<MOE_FP8_E4M3> {
  i32x8 v;  // two 16-byte chunks, consecutive registers as the MFMA wants them
  static constexpr int kKBytes = 64;
  static constexpr int kReads = 2, kMfma = 1;
  template <int RB>
  __device__ __forceinline__ void load(const unsigned char* base, int row, int s, int half) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + lds_pos<RB>(row, 4 * s + 2 * half));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + lds_pos<RB>(row, 4 * s + 2 * half + 1));
    v = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
  }
  __device__ __forceinline__ static void mma(f32x16& c, const Frag& a, const Frag& b) {
    // formats 0/0 = E4M3 x E4M3; E8M0 scales of 127 = 1.0
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, b.v, c, 0, 0, 0, 127, 0, 127);
  }
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// One work item: expert, first row / column, valid row end, and where its A
// and B rows live; K slabs [kb, kb + nk) of the tile.
struct Tile {
  int e, row0, row_end, n0, nk, rowB;
  int kb;     // first K slab of this work item
  int split;  // -1: whole tile; else the split index (last round only)
  int kr;     // SchedKR: the expert's rows (K extent)
  size_t a_off, a_bytes, b_off, b_bytes;
};

// Buffer descriptors of a tile's A rows and B rows: reads past the end of
// the A or B array return zero (ragged M tail, N tail, empty experts).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t off, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(static_cast<const unsigned char*>(base) + off), (short)0,
      int(bytes < 0x7FFFFFF0u ? bytes : 0x7FFFFFF0u), 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_ptr_t;

// Loader offsets of one lane for global row pitch rowB.  A 1 KB wave load
// fills 1024/RB rows of LDS with lane l at byte 16*l (row l/(RB/16),
// position l%(RB/16)), so the lane fetches the chunk that the swizzle keeps
// at that position.  With 128-byte rows the swizzle of a row group depends
// on the group's parity (e / o); with 64-byte rows it does not.
struct LoadOff {
  int e, o;
};
template <int RB>
__device__ __forceinline__ LoadOff load_off(int rowB, int lane) {
  constexpr int LPR = RB / 16, RPL = 1024 / RB, SW = 256 / RB;
  const int r = lane / LPR, p = lane % LPR;
  const int ce = p ^ ((r / SW) % LPR), co = p ^ (((r + RPL) / SW) % LPR);
  return LoadOff{r * rowB + (ce << 4), r * rowB + (co << 4)};
}

// One K slab of A and B straight from memory into LDS stage `st`: wave w
// fills row groups w*GA .. w*GA+GA-1 of A and w*GB .. w*GB+GB-1 of B.
template <class C>
__device__ __forceinline__ void issue_slab(unsigned char* lds, int st, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, int wave, LoadOff lo,
                                           int rowB, int koff) {
  constexpr int RPL = C::kRowsPerLoad;
  unsigned char* A = lds + st * C::kStage + wave * C::kGA * 1024;
  unsigned char* B = lds + st * C::kStage + C::kAStage + wave * C::kGB * 1024;
  const int ga0 = wave * C::kGA, gb0 = wave * C::kGB;
#pragma unroll
  for (int i = 0; i < (C::kGA > C::kGB ? C::kGA : C::kGB); ++i) {
    if (i < C::kGA) {
      const int q = ga0 + i;
      const int v = ((q & 1) ? lo.o : lo.e) + q * RPL * rowB + koff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t*)(A + i * 1024), 16, v, 0, 0, 0);
    }
    if (i < C::kGB) {
      const int q = gb0 + i;
      const int v = ((q & 1) ? lo.o : lo.e) + q * RPL * rowB + koff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t*)(B + i * 1024), 16, v, 0, 0, 0);
    }
  }
}

// SchedKR stage layout: each operand's part holds the slab's 64 K rows, row
// k at k * 512 bytes (256 M- or N-columns of bf16).  The 16-byte chunk c of
// row k sits at chunk c ^ kr_swz(k % 4): a transpose read takes four rows of
// one 32-byte column pair per 16 lanes (and two neighbouring pairs per 32
// lanes), and the XOR puts those four rows at distinct 128-byte and 256-byte
// bank positions.
__device__ __forceinline__ int kr_swz(int k4) { return (0xCA60 >> (4 * k4)) & 15; }

// Loader offsets of one lane for a global row pitch: a 1 KB wave load fills
// two K rows (lane l: row l / 32, chunk position l % 32); e / o for a row
// pair of even / odd index (rows 4i, 4i+1 / 4i+2, 4i+3).
__device__ __forceinline__ LoadOff load_off_kr(int pitch, int lane) {
  const int r = lane >> 5, p = lane & 31;
  return LoadOff{r * pitch + ((p ^ kr_swz(r)) << 4), r * pitch + ((p ^ kr_swz(r + 2)) << 4)};
}

// One 64-row K slab of A and B into LDS stage `stage` (SchedKR): wave w fills
// K-row pairs w*GA .. w*GA+GA-1 of A and w*GB .. of B.  The descriptors cover
// this slab's rows only, starting at the tile's first column.
template <class C>
__device__ __forceinline__ void issue_slab_kr(unsigned char* stage, __amdgpu_buffer_rsrc_t ra,
                                              __amdgpu_buffer_rsrc_t rb, int wave, LoadOff la,
                                              LoadOff lb, int pa, int pb) {
  unsigned char* A = stage + wave * C::kGA * 1024;
  unsigned char* B = stage + C::kAStage + wave * C::kGB * 1024;
  const int ga0 = wave * C::kGA, gb0 = wave * C::kGB;
#pragma unroll
  for (int i = 0; i < (C::kGA > C::kGB ? C::kGA : C::kGB); ++i) {
    if (i < C::kGA) {
      const int q = ga0 + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t*)(A + i * 1024), 16, (q & 1) ? la.o : la.e,
                                               2 * q * pa, 0, 0);
    }
    if (i < C::kGB) {
      const int q = gb0 + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t*)(B + i * 1024), 16, (q & 1) ? lb.o : lb.e,
                                               2 * q * pb, 0, 0);
    }
  }
}

// SchedKR fragment of substep s: lane l needs columns (m) mb + l % 32 and K
// values 16 s + 8 (l / 32) + 0..7.  A transpose read hands 16 lanes a 4 x 16
// block: the lanes 4j .. 4j+3 of a 16-lane group address four consecutive
// columns of K row j, and lane i of the group receives column i of the four
// rows.  Two reads give K + 0..3 and K + 4..7.  `off` is the lane's byte
// offset inside the part for its column block (kr_lane_off), K row 0.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ int kr_lane_off(int mb, int lane) {
  const int sp = lane & 15, k4 = sp >> 2;
  const int col = mb + ((lane >> 4) & 1) * 16 + 4 * (sp & 3);
  return (8 * (lane >> 5) + k4) * 512 + (((col >> 3) ^ kr_swz(k4)) << 4) + (col & 7) * 2;
}
__device__ __forceinline__ void load_tr_frag(Frag<MOE_BF16>& f, const unsigned char* part, int off,
                                             int s) {
  const unsigned char* p = part + off + s * 16 * 512;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr_t*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr_t*)(p + 4 * 512));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  f.v = u32x4{a[0], a[1], b[0], b[1]};
}

// Fragments of substep s of one LDS stage (MI A and NJ B fragments per wave).
template <class C, int DT>
__device__ __forceinline__ void load_frags(Frag<DT> (&fa)[C::kMI], Frag<DT> (&fb)[C::kNJ],
                                           const unsigned char* As, int arow, int brow, int s,
                                           int half) {
#pragma unroll
  for (int i = 0; i < C::kMI; ++i) fa[i].template load<C::kRowB>(As, arow + i * 32, s, half);
#pragma unroll
  for (int j = 0; j < C::kNJ; ++j)
    fb[j].template load<C::kRowB>(As + C::kAStage, brow + j * 32, s, half);
}

template <class C, int DT>
__device__ __forceinline__ void mma_all(f32x16 (&acc)[C::kMI][C::kNJ], const Frag<DT> (&fa)[C::kMI],
                                        const Frag<DT> (&fb)[C::kNJ]) {
#pragma unroll
  for (int i = 0; i < C::kMI; ++i)
#pragma unroll
    for (int j = 0; j < C::kNJ; ++j) Frag<DT>::mma(acc[i][j], fa[i], fb[j]);
}

// Single-buffered fragments (fp8, whose 8-register fragments and
// VGPR-resident accumulators leave no room for a second set): multiply,
// and reload each fragment for substep s of stage As right after its last
// MFMA.  B fragments go first (j outer), so the next substep's first MFMAs
// find theirs loaded early.
template <class C, int DT, bool reload>
__device__ __forceinline__ void mma_reload(f32x16 (&acc)[C::kMI][C::kNJ], Frag<DT> (&fa)[C::kMI],
                                           Frag<DT> (&fb)[C::kNJ], const unsigned char* As,
                                           int arow, int brow, int s, int half) {
#pragma unroll
  for (int j = 0; j < C::kNJ; ++j) {
#pragma unroll
    for (int i = 0; i < C::kMI; ++i) {
      Frag<DT>::mma(acc[i][j], fa[i], fb[j]);
      if (j == C::kNJ - 1 && reload) fa[i].template load<C::kRowB>(As, arow + i * 32, s, half);
    }
    if (reload) fb[j].template load<C::kRowB>(As + C::kAStage, brow + j * 32, s, half);
  }
  // keep that order: a reload may only follow the last MFMA that reads the
  // fragment it replaces
  constexpr int R = Frag<DT>::kReads;
#pragma unroll
  for (int j = 0; j < C::kNJ; ++j) {
#pragma unroll
    for (int i = 0; i < C::kMI; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (j == C::kNJ - 1 && reload) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
    if (reload) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
}

// s_waitcnt: at most N vector-memory operations outstanding and no LDS read
// (lgkmcnt 0; expcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Row of accumulator register r of MFMA block i (relative to the wave's rows).
__device__ __forceinline__ int acc_row(int i, int r, int half) {
  return i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
}

template <class C, int DT, int MODE>
__device__ __forceinline__ void epilogue(const GemmArgs& g, f32x16 (&acc)[C::kMI][C::kNJ],
                                         const Tile& T, int wave, int wm, int wn, int half,
                                         int l32, unsigned char* free_lds) {
  constexpr int MI = C::kMI, NJ = C::kNJ;
  const int e = T.e, row0 = T.row0, row_end = T.row_end, n0 = T.n0;
  const int rbase = row0 + wm * (MI * 32);   // the wave's first row
  const int cbase = n0 + wn * (NJ * 32);     // the wave's first column
  const int wrow = __builtin_amdgcn_readfirstlane(wm * (MI * 32));  // the same, relative to the tile
  const int nrow = row_end - row0 < C::kBM ? row_end - row0 : C::kBM;  // rows of the tile
  if (MODE == kModeFC1) {
    static_assert(MODE != kModeFC1 || NJ % 2 == 0, "FC1 pairs gate and up blocks");
    const int hf = g.N / 2;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float rmax[16];
#pragma unroll
      for (int p = 0; p < NJ / 2; ++p) {
        const int ch = cbase / 2 + p * 32 + l32;
        const int colg = cbase + (2 * p) * 32 + l32;  // packed column of G
        float sg = 1.f, su = 1.f;
        if (DT == MOE_FP8_E4M3) {
          sg = g.b_scale[size_t(e) * g.N + colg];
          su = g.b_scale[size_t(e) * g.N + colg + 32];
        }
        if constexpr (DT == MOE_BF16) {
          // Buffer stores: the row offset (uniform in the wave) goes in the
          // scalar offset, the lane's column in the vector offset, and the
          // descriptors end at the expert's last row, so rows past it are
          // dropped without a compare and a branch per value (in place of a
          // 64-bit address per value: Mixtral-shaped FC1 3.47 -> 3.41 ms; with
          // the same change in the FC2, dA and weight-gradient epilogues the
          // DeepSeekMoE-shaped training step 7.39 -> 7.30 ms).  A is stored
          // rounded to bf16, so the hardware reciprocal (1 ulp) replaces the
          // division (Mixtral-shaped FC1 -0.6%).
          const int rowa = hf * 2, rows = g.N * 2;
          const __amdgpu_buffer_rsrc_t ra = rsrc(g.out, size_t(row0) * rowa, size_t(nrow) * rowa);
          const __amdgpu_buffer_rsrc_t rs =
              rsrc(g.save ? g.save : g.out, size_t(row0) * rows, g.save ? size_t(nrow) * rows : 0);
          const int va = 4 * half * rowa + ch * 2, vs = 4 * half * rows + colg * 2;
          auto stores = [&](auto keep) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int srow = wrow + acc_row(i, r, 0);  // the lane's row, less 4 * half
              const float G = acc[i][2 * p][r], U = acc[i][2 * p + 1][r];
              const float a = G * __builtin_amdgcn_rcpf(1.0f + __expf(-G)) * U;
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(a)), ra, va, srow * rowa, 0);
              if constexpr (decltype(keep)::value) {
                // G|U kept for the backward, read again only there:
                // nontemporal stores (DeepSeekMoE-shaped FC1 -2%)
                __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(G)), rs, vs, srow * rows, 2);
                __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(U)), rs, vs + 64, srow * rows, 2);
              }
            }
          };
          if (g.save) stores(std::true_type{});
          else stores(std::false_type{});
          continue;
        }
        // FP8 and fp32: fp32 A through the same buffer stores; FP8 reads each
        // row's scale through a descriptor ending at the expert too, so a row
        // past it has scale 0, A = 0 and adds nothing to the row maxima
        const int rowa = hf * 4, rows = g.N * 2;
        const __amdgpu_buffer_rsrc_t ra = rsrc(g.out, size_t(row0) * rowa, size_t(nrow) * rowa);
        const __amdgpu_buffer_rsrc_t rs =
            rsrc(g.save ? g.save : g.out, size_t(row0) * rows, g.save ? size_t(nrow) * rows : 0);
        const __amdgpu_buffer_rsrc_t rx = rsrc(DT == MOE_FP8_E4M3 ? static_cast<const void*>(g.a_scale) : g.out,
                                               size_t(row0) * 4, DT == MOE_FP8_E4M3 ? size_t(nrow) * 4 : 0);
        const int va = 4 * half * rowa + ch * 4, vs = 4 * half * rows + colg * 2, vx = 4 * half * 4;
        auto rows_out = [&](auto keep) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int srow = wrow + acc_row(i, r, 0);  // the lane's row, less 4 * half
            float G = acc[i][2 * p][r], U = acc[i][2 * p + 1][r];
            if (DT == MOE_FP8_E4M3) {
              const float xs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, vx, srow * 4, 0));
              G *= xs * sg;
              U *= xs * su;
            }
            // fp32 A, which FP8 quantizes per row: the correctly rounded division
            const float a = silu_f(G) * U;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), ra, va, srow * rowa, 0);
            if (DT == MOE_FP8_E4M3) rmax[r] = p == 0 ? fabsf(a) : fmaxf(rmax[r], fabsf(a));
            if constexpr (decltype(keep)::value) {
              // G|U kept for the backward, read again only there: nontemporal
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(G)), rs, vs, srow * rows, 2);
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(U)), rs, vs + 64, srow * rows, 2);
            }
          }
        };
        if (g.save) rows_out(std::true_type{});
        else rows_out(std::false_type{});
      }
      if (DT == MOE_FP8_E4M3) {
        // row max over this wave's channels: reduce over the 32 lanes of a
        // half, then park it in the idle LDS stage ([wave column][tile row])
        float* red = reinterpret_cast<float*>(free_lds);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float m = rmax[r];
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          if (l32 == 0) red[wn * C::kBM + wm * (MI * 32) + acc_row(i, r, half)] = m;
        }
      }
    }
    if (DT == MOE_FP8_E4M3) {
      // the tile's row maxima over its channels: one plain store per row into
      // this column tile's slot (every slot has exactly one writer, so no
      // atomics and no reset); the quantization takes the max over slots.
      // The idle stage is read here and refilled by the next tile's loads.
      __syncthreads();
      const float* red = reinterpret_cast<const float*>(free_lds);
      const int ntn = (g.N + C::kBN - 1) / C::kBN;
      for (int q = threadIdx.x; q < C::kBM; q += C::kThreads) {
        float m = red[q];
#pragma unroll
        for (int w = 1; w < C::kWN; ++w) m = fmaxf(m, red[w * C::kBM + q]);
        const int row = row0 + q;
        if (row < row_end) g.row_amax[size_t(row) * ntn + n0 / C::kBN] = m;
      }
      __syncthreads();
    }
  } else if (MODE == kModeFC2) {
    // buffer stores as in FC1: row offset scalar, column per lane, rows past
    // the expert dropped by the descriptor (FP8: their scales read 0)
    const bool f32o = DT == MOE_F32 || g.out_f32;
    const int rowb = g.N * (f32o ? 4 : 2);
    const __amdgpu_buffer_rsrc_t ro = rsrc(g.out, size_t(row0) * rowb, size_t(nrow) * rowb);
    const __amdgpu_buffer_rsrc_t rx = rsrc(DT == MOE_FP8_E4M3 ? static_cast<const void*>(g.a_scale) : g.out,
                                           size_t(row0) * 4, DT == MOE_FP8_E4M3 ? size_t(nrow) * 4 : 0);
    const int vx = 4 * half * 4;
    auto stores = [&](auto f32c) {
      constexpr bool F = decltype(f32c)::value;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = cbase + j * 32 + l32;
        if (col >= g.N) continue;
        const int vo = 4 * half * rowb + col * (F ? 4 : 2);
        float cs = 1.f;
        if (DT == MOE_FP8_E4M3) cs = g.b_scale[size_t(e) * g.N + col];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int so = (wrow + acc_row(i, r, 0)) * rowb;
            float y = acc[i][j][r];
            if (DT == MOE_FP8_E4M3)
              y *= __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, vx, (wrow + acc_row(i, r, 0)) * 4, 0)) * cs;
            if constexpr (F)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), ro, vo, so, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(y)), ro, vo, so, 0);
          }
      }
    };
    if (f32o) stores(std::true_type{});
    else stores(std::false_type{});
  } else if (MODE == kModeBwdDA) {
    // dA tile -> dG, dU (packed like the forward's G|U) and A = SiLU(G)*U.
    // For each 32-channel block j, the kept G|U of the wave's rows (64 packed
    // columns, 128 B per row) go global -> LDS (the stage that is idle during
    // the epilogue, split evenly over the waves) in direct loads, a chunk of
    // rows at a time, then come out of LDS as needed.
    constexpr int kRegion = C::kStage / C::kNW;              // bytes of LDS per wave
    constexpr int kRows = (kRegion / 128 < MI * 32 ? kRegion / 128 : MI * 32) / 32 * 32;  // whole blocks
    constexpr int kIPer = kRows / 32;                        // MFMA blocks per chunk
    static_assert(kIPer >= 1 && MI % kIPer == 0, "chunk of whole MFMA blocks");
    const int hf = g.N;
    const size_t rowb = size_t(2 * hf) * 2;  // bytes per G|U row
    unsigned char* wl = free_lds + wave * kRegion;
    const uint16_t* wl16 = reinterpret_cast<const uint16_t*>(wl);
    const int lane = half * 32 + l32;
    // FP8: the per-expert column maxima of the stored values, which the
    // weight gradients' per-channel quantization needs, taken here instead
    // of in a pass over the stored arrays (DeepSeekMoE-shaped FP8 step: the
    // quantizing transposes 0.86 -> 0.74 ms, this epilogue +0.03 ms)
    const bool cmax = DT == MOE_FP8_E4M3 && g.row_amax != nullptr;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {                 // unrolled: acc stays in registers
      const int fb0 = cbase + j * 32;              // first channel of the group
      const int pb = (fb0 >> 5) * 64;              // its first packed column
      const int f = fb0 + l32;
      const int pg = pb + l32;
      float mg = 0.f, mu = 0.f, ma = 0.f;          // max |dG|, |dU|, |A| of the lane's rows
#pragma unroll
      for (int ic = 0; ic < MI / kIPer; ++ic) {
        const int crow0 = rbase + ic * kRows;
        // rows past the expert's last read as zero (their outputs are dropped
        // by the store descriptors, and A = SiLU(0) * 0 adds nothing to the
        // column maxima)
        const int gend = row0 + nrow;
        const __amdgpu_buffer_rsrc_t gsrc = rsrc(
            g.save, size_t(crow0) * rowb, size_t(gend > crow0 ? gend - crow0 : 0) * rowb);
        __builtin_amdgcn_s_waitcnt(0);             // earlier reads of this region done
#pragma unroll
        for (int q = 0; q < kRows / 8; ++q) {
          const int v = (q * 8 + (lane >> 3)) * int(rowb) + pb * 2 + (lane & 7) * 16;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(gsrc, (lds_ptr_t*)(wl + q * 1024), 16, v, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (f >= hf) continue;
        {
          // buffer stores (row offset scalar, column per lane, rows past the
          // expert dropped by the descriptors), as in the forward epilogues;
          // FP8 reads the rows' scales the same way
          const int rgu = 4 * hf, ra = 2 * hf;  // bytes per dG|dU row, per A row
          const __amdgpu_buffer_rsrc_t dgr = rsrc(g.out, size_t(row0) * rgu, size_t(nrow) * rgu);
          const __amdgpu_buffer_rsrc_t ar = rsrc(g.out2, size_t(row0) * ra, size_t(nrow) * ra);
          const __amdgpu_buffer_rsrc_t rx =
              rsrc(DT == MOE_FP8_E4M3 ? static_cast<const void*>(g.a_scale) : g.out, size_t(row0) * 4,
                   DT == MOE_FP8_E4M3 ? size_t(nrow) * 4 : 0);
          const float bs = DT == MOE_FP8_E4M3 ? g.b_scale[size_t(e) * g.N + f] : 1.f;
          const int vg = 4 * half * rgu + pg * 2, vaa = 4 * half * ra + f * 2;
#pragma unroll
          for (int ii = 0; ii < kIPer; ++ii) {
            const int i = ic * kIPer + ii;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int rl = acc_row(ii, r, half);   // row inside the chunk
              const int srow = wrow + ic * kRows + acc_row(ii, r, 0);  // tile row, less 4 * half
              const float G = bf16_to_f32(wl16[rl * 64 + l32]), U = bf16_to_f32(wl16[rl * 64 + 32 + l32]);
              const float sg = 1.0f / (1.0f + __expf(-G));
              const float si = G * sg;
              float dA = acc[i][j][r];
              if (DT == MOE_FP8_E4M3)
                dA *= __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, 4 * half * 4, srow * 4, 0)) * bs;
              const float vdg = dA * U * sg * (1.0f + G * (1.0f - sg)), vdu = dA * si, va = si * U;
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(vdg)), dgr, vg, srow * rgu, 0);
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(vdu)), dgr, vg + 64,
                                                    srow * rgu, 0);
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(va)), ar, vaa, srow * ra, 0);
              if (cmax) {
                // rows past the expert: dA = 0 and G|U read as zero, so all
                // three are zero there
                mg = fmaxf(mg, fabsf(vdg));
                mu = fmaxf(mu, fabsf(vdu));
                ma = fmaxf(ma, fabsf(va));
              }
            }
          }
        }
      }
      if (cmax) {
        // the two halves of the wave hold the same channels' other rows.
        // Rounding to bf16 is monotone and symmetric, so bf16(max |v|) is the
        // max of the stored |bf16(v)|; non-negative floats order as their
        // bit patterns, so an integer atomic max on the bits takes the max
        mg = fmaxf(mg, __shfl_xor(mg, 32, 64));
        mu = fmaxf(mu, __shfl_xor(mu, 32, 64));
        ma = fmaxf(ma, __shfl_xor(ma, 32, 64));
        if (half == 0 && f < hf) {
          unsigned* ca = reinterpret_cast<unsigned*>(g.row_amax) + size_t(e) * hf;
          unsigned* cg = reinterpret_cast<unsigned*>(g.row_amax) + size_t(g.E) * hf + size_t(e) * 2 * hf;
          atomicMax(ca + f, f32_to_bf16_bits(ma) << 16);
          atomicMax(cg + pg, f32_to_bf16_bits(mg) << 16);
          atomicMax(cg + pg + 32, f32_to_bf16_bits(mu) << 16);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // the idle stage is refilled by the next tile's loads
  } else {
    // weight gradients, fp32: rows m of expert e's [M][N] (DW13: N packed,
    // 32-column blocks alternating dW1 / dW3, so the target is uniform per
    // block); buffer stores as in the forward epilogues, FP8 reading the
    // per-expert channel scales of both transposed operands
    const int ld = MODE == kModeDW13 ? g.N / 2 : g.N;
    const int rowb = ld * 4;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = cbase + j * 32 + l32;
      if (n >= g.N) continue;
      const int nb = (cbase >> 5) + j;  // 32-column block
      const void* dst = (MODE == kModeDW13 && (nb & 1)) ? g.out2 : g.out;
      const int col = MODE == kModeDW13 ? (nb >> 1) * 32 + l32 : n;
      const __amdgpu_buffer_rsrc_t ro = rsrc(dst, (size_t(e) * g.M + row0) * rowb, size_t(nrow) * rowb);
      const __amdgpu_buffer_rsrc_t rx =
          rsrc(DT == MOE_FP8_E4M3 ? static_cast<const void*>(g.a_scale) : dst, (size_t(e) * g.M + row0) * 4,
               DT == MOE_FP8_E4M3 ? size_t(nrow) * 4 : 0);
      const float bs = DT == MOE_FP8_E4M3 ? g.b_scale[size_t(e) * g.N + n] : 1.f;
      const int vo = 4 * half * rowb + col * 4;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = acc[i][j][r];
          if (DT == MOE_FP8_E4M3)
            v *= __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, 4 * half * 4, (wrow + acc_row(i, r, 0)) * 4, 0)) * bs;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ro, vo, (wrow + acc_row(i, r, 0)) * rowb, 0);
        }
    }
  }
}

// Split-K tail.  The tiles of a persistent grid's last, partial round are
// split along K so that every workgroup has work in it.  Each split stores
// its fp32 partial tile (1 KB per lane-row, coalesced); the split that
// arrives last on the tile's device-scope counter adds all partials in split
// order and goes on to the epilogue, so the sum does not depend on arrival
// order.  Returns true in the workgroup that finishes the tile.
template <class C>
__device__ __forceinline__ bool splitk_combine(const GemmArgs& g, f32x16 (&acc)[C::kMI][C::kNJ],
                                               int slot0, int f, int s, int cidx, int wave,
                                               int lane, int* flag) {
  constexpr int MI = C::kMI, NJ = C::kNJ;
  constexpr size_t kSlot = size_t(C::kBM) * C::kBN / 4;  // f32x4 per partial tile
  f32x4* base = reinterpret_cast<f32x4*>(g.part) + size_t(wave) * MI * NJ * 4 * 64 + lane;
  f32x4* mine = base + size_t(slot0 + s) * kSlot;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        mine[((i * NJ + j) * 4 + q) * 64] =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
  __threadfence();  // release: partial visible device-wide before the count
  __syncthreads();
  if (threadIdx.x == 0) *flag = atomicAdd(g.cnt + cidx, 1u) == unsigned(f - 1);
  __syncthreads();
  if (!*flag) return false;
  __threadfence();  // acquire: the other splits' partials
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int t = 0; t < f; ++t) {
    const f32x4* p = base + size_t(slot0 + t) * kSlot;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = p[((i * NJ + j) * 4 + q) * 64];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[i][j][4 * q + c] += v[c];
        }
  }
  return true;
}

template <class C, int DT, int MODE, int SCHED>
__global__ void __launch_bounds__(C::kThreads, C::kWavesPerSimd) grouped_gemm_kernel(GemmArgs g) {
  constexpr int BM = C::kBM, BN = C::kBN, MI = C::kMI, NJ = C::kNJ;
  constexpr int RB = C::kRowB, NS = C::kStages, D = NS - 1;  // D slabs in flight ahead
  extern __shared__ __align__(16) unsigned char lds[];
  // SchedKR keeps its two stages in arrays of their own and runs the K loop
  // with the stage parity known at compile time: the compiler can then tell
  // that a transpose read of one stage does not touch the slab the LDS-DMA
  // loads are filling in the other (through one array, with a run-time
  // offset, it waits for every load in flight before each transpose read).
  constexpr int KRS = SCHED == kSchedKR ? C::kStage : 16;
  __shared__ __align__(16) unsigned char kr0[KRS];
  __shared__ __align__(16) unsigned char kr1[KRS];
  __shared__ int tpre[MOE_MAX_EXPERTS + 1];  // tiles before expert e
  __shared__ int offs[MOE_MAX_EXPERTS + 1];  // SchedM / KR: row offsets; SchedK: padded K prefix
  __shared__ int split_flag;
  constexpr int EB = Elem<DT>::bytes;
  constexpr bool ARR = MODE == kModeFC1Arr;
  constexpr int EMODE = ARR ? kModeFC1 : MODE;  // the epilogue's mode
  static_assert(!ARR || (SCHED == kSchedM && DT == MOE_BF16), "tile arrival: bf16 FC1");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / C::kWN, wn = wave % C::kWN;
  const int half = lane >> 5, l32 = lane & 31;
  const int NT = ceil_div(g.N, BN);
  const int MT = SCHED != kSchedM ? ceil_div(g.M, BM) : 0;
  static_assert(SCHED != kSchedKR || (DT == MOE_BF16 && RB == 128 && BM == 256 && BN == 256 && NS == 2),
                "SchedKR: bf16, 64-row slabs of 512-byte LDS rows, two stages");

  for (int e = tid; e <= g.E; e += C::kThreads) {
    int o = g.offsets[e];
    offs[e] = o < 0 ? 0 : (o > g.rows ? g.rows : o);  // never address past `rows`
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0, kp = 0, prev = offs[0];
    tpre[0] = 0;
    for (int e = 0; e < g.E; ++e) {
      int lo = prev, hi = offs[e + 1] < prev ? prev : offs[e + 1];
      prev = hi;
      if (SCHED == kSchedM) {
        offs[e + 1] = hi;
        run += ceil_div(hi - lo, BM) * NT;
      } else if (SCHED == kSchedKR) {
        offs[e + 1] = hi;
        run += MT * NT;
      } else {
        offs[e] = kp;  // becomes the padded K prefix
        kp += ceil_div(hi - lo, kpad_elems<DT>()) * kpad_elems<DT>();
        run += MT * NT;
      }
      tpre[e + 1] = run;
    }
    if (SCHED == kSchedK) offs[g.E] = kp;
  }
  __syncthreads();
  const int total = __builtin_amdgcn_readfirstlane(tpre[g.E]);
  const int G = gridDim.x;
  const int b = blockIdx.x;
  // Work items: tiles [0, full) whole, then each of the last `rem` tiles as
  // f K splits (f = 1: no split).
  int full = total, f = 1;
  if (g.part != nullptr && total % G != 0) {
    const int rem = total % G;
    f = G / rem < kMaxSplit ? G / rem : kMaxSplit;
    if (SCHED == kSchedM) {
      const int nkm = g.K * EB / RB;
      if (f > nkm) f = nkm > 1 ? nkm : 1;
    }
    if (f > 1) full = total - rem;
    else f = 1;
  }
  const int work = full + (total - full) * f;
  // the workgroups of one XCD (b % 8) take consecutive work items
  int t = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  if (t >= work) return;

  // LDS values read here are the same in every lane: keep them in scalar
  // registers, so the work-item state costs no vector registers.
  auto sld = [](const int* p) { return __builtin_amdgcn_readfirstlane(*p); };
  auto tile_of = [&](int tt) {
    int lo = 0, hi = g.E - 1;  // expert e with tpre[e] <= tt < tpre[e+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sld(tpre + mid) <= tt) lo = mid; else hi = mid - 1;
    }
    Tile T;
    T.e = lo;
    T.kr = 0;
    const int local = tt - sld(tpre + lo);
    const int o0 = sld(offs + lo), o1 = sld(offs + lo + 1);
    if (SCHED == kSchedM) {
      // experts in order, m-tiles fastest: consecutive tiles share a weight block
      const int mt_e = ceil_div(o1 - o0, BM);
      const int nt = local / mt_e, mt = local - nt * mt_e;
      T.row0 = o0 + mt * BM;
      T.row_end = o1;
      T.n0 = nt * BN;
      T.rowB = g.K * EB;
      T.a_off = size_t(T.row0) * T.rowB;
      // rows past the expert's last read as zero without touching memory (a
      // ragged row tile then fetches only its own rows: Mixtral-shaped FC1
      // -2.6%, 352B-shaped with Zipf routing -3.8%)
      T.a_bytes = size_t(o1 - T.row0) * T.rowB;
      T.b_off = (size_t(lo) * g.N + T.n0) * T.rowB;
    } else if (SCHED == kSchedKR) {
      // m-tiles fastest: consecutive tiles share the expert's B columns
      const int nt = local / MT, mt = local - nt * MT;
      T.row0 = mt * BM;
      T.row_end = g.M;
      T.n0 = nt * BN;
      T.rowB = 0;
      T.kr = o1 - o0;
      T.a_off = size_t(o0) * g.M * 2 + size_t(T.row0) * 2;
      T.b_off = size_t(o0) * g.N * 2 + size_t(T.n0) * 2;
      T.a_bytes = T.b_bytes = 0;
      T.nk = ceil_div(T.kr, 64);
      T.kb = 0;
      T.split = -1;
      return T;
    } else {
      const int nt = local / MT, mt = local - nt * MT;
      const int k0 = o0, ke = o1 - o0;
      T.row0 = mt * BM;
      T.row_end = g.M;
      T.n0 = nt * BN;
      T.rowB = ke * EB;
      T.a_off = size_t(k0) * g.M * EB + size_t(T.row0) * T.rowB;
      T.a_bytes = size_t(g.M - T.row0) * T.rowB;
      T.b_off = size_t(k0) * g.N * EB + size_t(T.n0) * T.rowB;
    }
    T.b_bytes = size_t(g.N - T.n0) * T.rowB;
    T.nk = T.rowB / RB;
    T.kb = 0;
    T.split = -1;
    return T;
  };
  auto item_of = [&](int w) {
    if (w < full) return tile_of(w);
    const int u = w - full, s = u % f;
    Tile T = tile_of(full + u / f);
    const int k0 = s * T.nk / f, k1 = (s + 1) * T.nk / f;
    T.kb = k0;
    T.nk = k1 - k0;
    T.split = s;
    return T;
  };

  constexpr int S = RB / Frag<DT>::kKBytes;             // substeps per slab
  static_assert(S >= 2 && S % 2 == 0, "fragment double buffer needs an even substep count");
  constexpr int NR = (MI + NJ) * (SCHED == kSchedKR ? 2 : Frag<DT>::kReads);  // LDS reads per substep
  constexpr int NM = MI * NJ * Frag<DT>::kMfma;         // MFMAs per substep
  constexpr int NV = C::kGA + C::kGB;                   // global loads per slab per wave
  constexpr bool kSingle = Frag<DT>::kReads == 2;       // fp8: single-buffered fragments
  // fragment rows inside a stage
  const int arow = wm * (MI * 32) + l32, brow = wn * (NJ * 32) + l32;
  // SchedKR: the lane's transpose-read offsets of its column blocks
  int kra[SCHED == kSchedKR ? MI : 1], krb[SCHED == kSchedKR ? NJ : 1];
  if (SCHED == kSchedKR) {
#pragma unroll
    for (int i = 0; i < MI; ++i) kra[i] = kr_lane_off(wm * (MI * 32) + i * 32, lane);
#pragma unroll
    for (int j = 0; j < NJ; ++j) krb[j] = kr_lane_off(wn * (NJ * 32) + j * 32, lane);
  }
  auto frags = [&](Frag<DT>(&fa)[MI], Frag<DT>(&fb)[NJ], const unsigned char* st, int s) {
    if constexpr (SCHED == kSchedKR) {
#pragma unroll
      for (int i = 0; i < MI; ++i) load_tr_frag(fa[i], st, kra[i], s);
#pragma unroll
      for (int j = 0; j < NJ; ++j) load_tr_frag(fb[j], st + C::kAStage, krb[j], s);
    } else {
      load_frags<C, DT>(fa, fb, st, arow, brow, s, half);
    }
  };

  // The slabs of this workgroup's work items form one stream; slab c of the
  // stream sits in stage c % NS.  The loader walks the same items as the
  // MFMAs, D slabs ahead, skipping items without K slabs.
  int lw = t, lk = 0, issued = 0;
  Tile lt = item_of(lw);
  bool ldone = false;
  while (lt.nk == 0) {
    lw += G;
    if (lw >= work) { ldone = true; break; }
    lt = item_of(lw);
  }
  __amdgpu_buffer_rsrc_t lra = rsrc(g.A, lt.a_off, lt.a_bytes), lrb = rsrc(g.B, lt.b_off, lt.b_bytes);
  LoadOff llo = load_off<RB>(lt.rowB, lane);
  // SchedKR: row pitches of A and B, the lanes' loader offsets
  const int pa = g.M * 2, pb = g.N * 2;
  const LoadOff kla = load_off_kr(pa, lane), klb = load_off_kr(pb, lane);
  // FC1Arr: before a row tile's first slab is loaded, wait until the
  // dispatch copy has released all rows of its expert (a bounded wait: thread 0
  // polls the counts, the workgroup meets it at a barrier, and sleeps between
  // polls), then acquire.  Once the copy has released every row no tile waits
  // again.  The poll's result goes through split_flag, which the split-K
  // combine uses only after a workgroup's last item has loaded its slabs.
  // Returns true once the copy has released every row.
  auto gate = [&](const Tile& T) -> bool {
    const uint32_t need = uint32_t(T.row_end - sld(offs + T.e));
    const uint32_t total = uint32_t(sld(offs + g.E));
    int f = 0;
    for (int it = 0;; ++it) {
      if (tid == 0) {
        const uint32_t r = __hip_atomic_load(g.ready + T.e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t d = __hip_atomic_load(g.done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        split_flag = (r >= need ? 1 : 0) | (d >= total ? 2 : 0);
      }
      __syncthreads();
      f = split_flag;
      __syncthreads();
      if (f) break;
      if (it >= g.spin_limit) {  // 2^20 polls, ~0.5 s: the copy is not running beside this kernel
        if (tid == 0) atomicOr(g.status, 1);
        f = 2;
        break;
      }
      __builtin_amdgcn_s_sleep(16);
    }
    // acquire only (agent scope): drop stale lines, no write-back of this
    // XCD's dirty lines
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return (f & 2) != 0;
  };
  bool all_ready = !ARR;
  if constexpr (ARR) {
    if (!ldone) all_ready = gate(lt);
  }
  // kdst: the stage SchedKR's slab goes to (slab `issued` of the stream)
  auto issue = [&](unsigned char* kdst) {
    if (ldone) return;
    if (SCHED == kSchedKR) {
      // descriptors of this slab's rows: rows past the expert's end, and
      // columns past the last row's end, read as zeros
      const int k0 = (lt.kb + lk) * 64, nr = lt.kr - k0 < 64 ? lt.kr - k0 : 64;
      const __amdgpu_buffer_rsrc_t ra =
          rsrc(g.A, lt.a_off + size_t(k0) * pa, size_t(nr) * pa - size_t(lt.row0) * 2);
      const __amdgpu_buffer_rsrc_t rb =
          rsrc(g.B, lt.b_off + size_t(k0) * pb, size_t(nr) * pb - size_t(lt.n0) * 2);
      issue_slab_kr<C>(kdst, ra, rb, wave, kla, klb, pa, pb);
    } else {
      issue_slab<C>(lds, issued % NS, lra, lrb, wave, llo, lt.rowB, (lt.kb + lk) * RB);
    }
    ++issued;
    if (++lk < lt.nk) return;
    lk = 0;
    do {
      lw += G;
      if (lw >= work) { ldone = true; return; }
      lt = item_of(lw);
    } while (lt.nk == 0);
    if (SCHED != kSchedKR) {
      lra = rsrc(g.A, lt.a_off, lt.a_bytes);
      lrb = rsrc(g.B, lt.b_off, lt.b_bytes);
      llo = load_off<RB>(lt.rowB, lane);
    }
    if constexpr (ARR) {
      if (!all_ready) all_ready = gate(lt);
    }
  };
  // wait until slab c has landed: n = slabs issued after it (in flight)
  auto wait_slab = [&](int c) {
    const int n = issued - 1 - c;
    if (D >= 3 && n >= 2) wait_vm_lds<(D >= 3 ? 2 * NV : 0)>();
    else if (D >= 2 && n >= 1) wait_vm_lds<(D >= 2 ? NV : 0)>();
    else wait_vm_lds<0>();
  };

  // stage i of the ring; SchedKR's two stages are its own arrays
  auto stage = [&](int i) -> unsigned char* {
    if constexpr (SCHED == kSchedKR) return i ? kr1 : kr0;
    else return lds + i * C::kStage;
  };
  for (int i = 0; i < D; ++i) issue(stage(i));
  wait_slab(0);
  __syncthreads();
  Frag<DT> fa[2][MI], fb[2][NJ];
  if (issued > 0) frags(fa[0], fb[0], stage(0), 0);

  int c = 0;             // stream slab the MFMAs consume next
  bool drain = false;    // an epilogue's stores may be outstanding
  f32x16 acc[MI][NJ];    // the current item's accumulators
  bool mact = true;      // the current tile has rows in this wave's 128
  // One K slab: As is stage c % NS (holding slab c, fa[0]/fb[0] its first
  // fragments), Nx stage (c + 1) % NS.  SchedKR (two stages) loads slab c + 1
  // into Nx.
  auto kstep = [&](const unsigned char* As, unsigned char* Nx) {
    // Stores and loads share one counter and may complete out of order:
    // after an epilogue, drain it before counting loads again.
    if (drain) {
      __builtin_amdgcn_s_waitcnt(0);
      drain = false;
    }
    // slab c + D goes into the stage that slab c - 1 left (read out before
    // the last barrier)
    issue(Nx);
    // A wave whose rows of a ragged tile all lie past the expert's last row
    // (they read as zero) skips its MFMAs and their fragment reads; it still
    // issues its share of the loads and meets every barrier (Mixtral-shaped
    // FC1 -1.6%, 352B-shaped with Zipf routing -1%).
    if (SCHED == kSchedM && !mact) {
      wait_slab(c + 1);
      __syncthreads();
      if (c + 1 < issued) frags(fa[0], fb[0], Nx, 0);
      ++c;
      return;
    }
    if (kSingle) {
#pragma unroll
      for (int s = 0; s + 1 < S; ++s)
        mma_reload<C, DT, true>(acc, fa[0], fb[0], As, arow, brow, s + 1, half);
      wait_slab(c + 1);
      __syncthreads();
      if (c + 1 < issued)
        mma_reload<C, DT, true>(acc, fa[0], fb[0], Nx, arow, brow, 0, half);
      else
        mma_reload<C, DT, false>(acc, fa[0], fb[0], As, arow, brow, 0, half);
      ++c;
      return;
    }
    // The wave runs its MFMA substeps at raised issue priority, so where
    // both waves of a SIMD have instructions ready the one in its MFMA
    // phase goes first (Mixtral-shaped FC1 -1.5%, FC2 -0.7%); the barrier
    // wait, the next slab's first fragments and the load issue run at the
    // normal priority.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s + 1 < S; ++s) {
      frags(fa[(s + 1) & 1], fb[(s + 1) & 1], As, s + 1);
      mma_all<C, DT>(acc, fa[s & 1], fb[s & 1]);
    }
    // interleave: the substep's LDS reads spread over its MFMAs (and one
    // global load per MFMA early on)
#pragma unroll
    for (int s = 0; s + 1 < S; ++s)
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        constexpr int rq = NR / NM;
        if (rq > 0) __builtin_amdgcn_sched_group_barrier(0x100, rq, 0);
        if (q < NR % NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (s == 0 && q < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    __builtin_amdgcn_s_setprio(0);
    wait_slab(c + 1);  // this stage read out; slab c+1 landed
    __syncthreads();
    // next slab's first fragments load while the last substep multiplies
    if (c + 1 < issued) frags(fa[0], fb[0], Nx, 0);
    mma_all<C, DT>(acc, fa[1], fb[1]);
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    ++c;
  };
  while (true) {
    const Tile cur = item_of(t);
    mact = SCHED != kSchedM || cur.row0 + wm * (MI * 32) < cur.row_end;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if constexpr (SCHED == kSchedKR) {
      // stage parity known in each copy of the step: an odd first slab, then
      // pairs, then an even last slab (one step under a run-time parity
      // branch instead keeps both copies' fragments live and spills)
      int kt = 0;
      if ((c & 1) && cur.nk > 0) {
        kstep(kr1, kr0);
        kt = 1;
      }
      for (; kt + 1 < cur.nk; kt += 2) {
        kstep(kr0, kr1);
        kstep(kr1, kr0);
      }
      if (kt < cur.nk) kstep(kr0, kr1);
    } else {
      for (int kt = 0; kt < cur.nk; ++kt) kstep(stage(c % NS), stage((c + 1) % NS));
    }

    // A split is its workgroup's last item: only the one that completes the
    // tile runs the epilogue.  Stage (c - 1) % NS holds no slab in flight.
    if (cur.split < 0 || splitk_combine<C>(g, acc, ((t - full) / f) * f, f, cur.split,
                                           (t - full) / f, wave, lane, &split_flag))
      epilogue<C, DT, EMODE>(g, acc, cur, wave, wm, wn, half, l32,
                            stage((c + NS - 1) % NS));
    drain = true;
    t += G;
    if (t >= work) break;
  }
}

}  // namespace moe

namespace moe_launch {

// Persistent launch: OCC workgroups per CU (fewer if there are fewer tiles).
// The tile count bound needs no device data: SchedM has at most
// ceil(rows/BM) + E row tiles, SchedK exactly E ceil(M/BM).
template <int>
__global__ void zero_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Bytes of split-K workspace a configuration needs (partial tiles + counters).
static_assert(moe::CfgFor<MOE_BF16>::type::kBM * moe::CfgFor<MOE_BF16>::type::kBN ==
                  moe::CfgFor<MOE_FP8_E4M3>::type::kBM * moe::CfgFor<MOE_FP8_E4M3>::type::kBN,
              "one split-K workspace size for every dtype");
template <class C>
constexpr size_t splitk_ws_bytes() {
  return size_t(moe::kMaxGrid) * C::kBM * C::kBN * 4 + size_t(moe::kMaxGrid) * 4;
}
template <class C>
inline void splitk_ws_set(moe::GemmArgs& a, void* ws) {
  a.part = static_cast<float*>(ws);
  a.cnt = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(ws) +
                                      size_t(moe::kMaxGrid) * C::kBM * C::kBN * 4);
}

template <class C, int DT, int MODE, int SCHED>
inline int launch_gemm(const moe::GemmArgs& a, int timer, hipStream_t s) {
  using namespace moe;
  // SchedKR's stages are static arrays of the kernel
  constexpr size_t dyn = SCHED == kSchedKR ? 0 : C::kLds;
  static bool attr = allow_lds(grouped_gemm_kernel<C, DT, MODE, SCHED>, dyn);
  if (!attr) return MOE_ERR_HIP;
  long grid = long(num_cus()) * C::kOcc;
  if (grid > kMaxGrid) grid = kMaxGrid;
  if (a.part == nullptr) {
    // without split-K, no more workgroups than tiles
    const long mt = SCHED == kSchedM ? (long(a.rows) + C::kBM - 1) / C::kBM + a.E
                                     : long(a.E) * ((a.M + C::kBM - 1) / C::kBM);
    const long tiles = mt * ((a.N + C::kBN - 1) / C::kBN);
    if (tiles < grid) grid = tiles;
  }
  if (grid < 1) grid = 1;
  timer_begin(timer, s);
  if (a.part != nullptr)
    hipLaunchKernelGGL(zero_u32_kernel<0>, dim3(1), dim3(kMaxGrid), 0, s, a.cnt, int(kMaxGrid));
  hipLaunchKernelGGL((grouped_gemm_kernel<C, DT, MODE, SCHED>), dim3(unsigned(grid)),
                     dim3(C::kThreads), dyn, s, a);
  timer_end(timer, s);
  return launch_status();
}

}  // namespace moe_launch
