// Grouped expert GEMM for experts with many rows (the prefill regime), gfx950.
//
// C[r][n] = act(sum_k A[arow(r)][k] * B_g[n][k]) for the rows r of each
// expert g (rows g_off[g] .. g_off[g+1] of the expert-grouped order), bf16
// operands and output, fp32 accumulation.  FC1 gathers its A rows through
// a_rows (the dispatch permutation token_of); FC2 reads the grouped rows
// in place.
//
// Work items are (expert, row tile, 256-column tile).  An expert's rows are
// cut into tiles of 256; its last tile is 256, 128 or 64 rows high, the
// smallest that holds what is left, so that skewed loads (many experts with
// a few dozen rows, a few with thousands) spend little MFMA work on padding
// rows.  Every tile is computed by 2 x 4 waves: 128 x 64 each (64 x 64 or
// 32 x 64 in the shorter tiles) in 32x32x16 bf16 MFMA blocks.  One
// workgroup of eight waves (two per SIMD, so that one wave's MFMAs run while
// the other waits on a load, a barrier or its epilogue) runs per compute
// unit and walks its items (a persistent grid); each XCD takes a contiguous
// range of items, so the column tiles of a row tile (which share its A
// rows) and the row tiles of an expert (which share its weights) run on the
// same L2 at about the same time.  The expert offsets sit in LDS, and a
// tile fetches the next tile's gathered row indices into LDS behind its own
// first loads, so that a tile starts without a dependent global load.
//
// K advances in stages of 32 elements through an LDS ring of four stage
// buffers filled by buffer loads in LDS mode (each lane 16 bytes, no
// register staging): three stages are in flight while one is multiplied.
// Every thread issues the same number of loads per stage (A rows past a
// short tile read zeros without a memory request), so "the next stage has
// landed" is an exact vmcnt wait, then one barrier per stage.  Fragment
// reads of the next k-step are issued at the front of each k-step, so they
// are complete when the stage ends.  LDS rows are 64 bytes (4 chunks);
// chunk c of row r sits at c ^ ((r >> 2) & 3), so the 32 lanes reading one
// fragment column touch distinct bank groups.
//
// A load instruction covers 16 rows x 64 bytes of a stage.  The load path
// pays per row (cache line) touched more than per byte, so two operand
// layouts put a stage's rows next to each other: B may come as the banded
// copy of the weights (b_bands: 256-row bands stored as 32-column blocks,
// so a weight tile's K stage is one contiguous 16 KB block), and FC1 writes
// H in 32-column blocks over all rows (c_kblock) that FC2 reads the same
// way (a_kblock).  Prefill FC1 / FC2: 1.68 / 1.64 ms row-major, 1.59 /
// 1.34 ms with both.
//
// Each lane ends with 4 consecutive output columns per block row (the
// MFMA computes the block transposed); one 32-row block row of the wave's
// columns at a time is activated, rounded to bf16, staged in LDS and
// stored as 128-byte row segments (stores straight from the accumulators,
// 16 bytes to each of 32 rows per instruction, took several times longer).
// The epilogue is kept short: buffer stores whose range ends at the tile's
// last row (no per-row test) and a one-instruction ReLU.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

constexpr int kGgNT = 512;                           // 8 waves, two per SIMD
constexpr int kGgNW = kGgNT / 64;
constexpr int kGgWN = 4;                             // waves along N (2 along M)
constexpr int kGgWCols = 256 / kGgWN;                // columns of a wave (64)
constexpr int kGgNJ = kGgWCols / 32;                 // 32-column blocks of a wave (2)
constexpr int kGgBN = 256;                           // columns per tile
constexpr int kGgBM = 256;                           // rows of a full tile
constexpr int kGgBKC = 4;                            // 16-byte chunks of K per row per stage
constexpr int kGgBK = kGgBKC * 8;                    // K elements per stage
constexpr int kGgNS = 4;                             // stage buffers in the ring
constexpr int kGgStage = (kGgBM + kGgBN) * kGgBKC;   // chunks per stage buffer (32 KB)
constexpr int kGgMaxG = 2048;

__device__ __forceinline__ int gg_swz(int r) { return (r >> 2) & 3; }

struct GgTile {
  int g;       // expert
  int row0;    // first grouped row
  int rows;    // rows of the expert in this tile (<= bm)
  int col0;    // first output column
};

typedef f32x16_t GgAcc[4][kGgNJ];

// Epilogue staging, one area per wave: a 32-row block row of the wave's
// 64 output columns in bf16 (rows padded by 16 bytes against bank
// conflicts), so that stores leave as 128-byte row segments.  The areas
// (8 x 4.5 KB) sit in the ring's last stage buffer and 4 KB past it: the
// next tile's first loads fill the other buffers, and the last buffer is
// next written after the barrier that every wave reaches only once its
// epilogue is done.
constexpr int kGgOutLd = kGgWCols + 8;              // bf16 elements per staged row
constexpr int kGgOutChunks = kGgNW * 32 * kGgOutLd * 2 / 16;
constexpr int kGgRingTail = kGgOutChunks > kGgStage ? kGgOutChunks - kGgStage : 0;
__shared__ u32x4 gg_ring[kGgNS * kGgStage + kGgRingTail];   // the LDS ring, 128 + 4 KB
// Source rows of a tile's A rows (FC1 gathers them through a_rows), double
// buffered: a tile reads its own and prefetches the next tile's.
__shared__ int gg_rows[2][kGgBM];

// One 16-byte chunk per lane from global memory straight into LDS (lane i
// writes bytes [16 i, 16 i + 16) after the wave-uniform LDS byte address
// lds).  Written as inline asm: the compiler's own form of this load makes
// it wait for every LDS-mode load in flight before any later LDS read it
// cannot prove disjoint, which would collapse the ring to one stage.  The
// ring's order is kept by the explicit vmcnt waits and barriers instead;
// the memory clobber keeps the loads in program order against the LDS
// reads.  M0 carries the LDS address (an operand: the compiler sets it).
__device__ __forceinline__ void gg_dma(BufRsrc r, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "{m0}"(lds)
               : "memory");
}

// One dword per lane into LDS (lane i writes bytes [4 i, 4 i + 4) after
// lds), as gg_dma.
__device__ __forceinline__ void gg_dma_dword(BufRsrc r, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "{m0}"(lds)
               : "memory");
}

// The 256 entries of a_rows from grouped row row0 on (past the end: zeros)
// into gg_rows[buf], one load per thread.
__device__ __forceinline__ void gg_fetch_rows(const GemmArgs& p, int total_rows, int row0, int buf,
                                              int wave, int lane) {
  const BufRsrc r = make_rsrc(p.a_rows, static_cast<uint64_t>(total_rows) * 4);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)&gg_rows[buf][wave * 64])));
  gg_dma_dword(r, lds, static_cast<uint32_t>(row0 + wave * 64 + lane) * 4u);
}

// One tile of height 64 * MI: main loop over K, then the epilogue.  The
// tile's source rows are in gg_rows[buf] (when A is gathered); next_row0 >= 0
// asks for the next tile's to be fetched into the other buffer.
template <int MI, int ACT, bool GATHER, bool DENSE>
__device__ __forceinline__ void gg_tile(const GemmArgs& p, const GgTile& t, int wave, int lane_in,
                                        GgAcc& acc, int buf, int next_row0, int total_rows) {
  // the lane index, opaque to the compiler per tile: the index arithmetic of
  // the three tile heights is then recomputed per tile instead of being
  // hoisted out of the tile loop (where it held registers the main loop
  // needs, and spilled); computed here by mbcnt (in asm, which the compiler
  // cannot hoist either), so that no register carries it between tiles
  (void)lane_in;
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  constexpr int BM = 64 * MI;
  constexpr int WM = BM / 2;                     // rows per wave
  // A rows loaded per stage: at least 128, so that every thread issues a
  // whole number of loads (rows past the tile read zeros, no memory request)
  constexpr int BMLD = BM < 128 ? 128 : BM;
  constexpr int ACH = BMLD * kGgBKC;             // A chunks per stage
  constexpr int NCH = ACH + kGgBN * kGgBKC;      // chunks loaded per stage
  constexpr int NDMA = NCH / kGgNT;              // loads per thread per stage
  static_assert(NCH % kGgNT == 0 && ACH % 64 == 0, "stage splits into wave loads");
  const int wm = wave / kGgWN, wn = wave % kGgWN;
  const int nk = p.K / kGgBK;

  const uint16_t* A = static_cast<const uint16_t*>(p.A);
  const uint16_t* B = static_cast<const uint16_t*>(p.B) + (int64_t)t.g * p.b_gstride;
  const uint64_t a_rows_total = static_cast<uint64_t>(p.a_nrows);
  const BufRsrc a_rsrc = make_rsrc(A, p.a_kblock > 0 ? static_cast<uint64_t>(p.a_kblock) * p.K * 2
                                                    : a_rows_total * p.lda * 2);
  const BufRsrc b_rsrc = make_rsrc(B, (uint64_t)p.N * p.ldb * 2);

  // this lane's chunk of each of its loads at K stage 0 (padding rows: an
  // offset past the buffer, which reads zeros)
  uint32_t d_off[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int q = (kGgNW * j + wave) * 64 + lane;
    if (q < ACH) {
      const int r = q / kGgBKC;
      const int c = (q % kGgBKC) ^ gg_swz(r);
      int64_t arow = -1;
      if (r < t.rows) arow = GATHER ? gg_rows[buf][r] : t.row0 + r;
      // row-major A: stage 0 of row arow; blocked A: the row's 64 bytes in block 0
      const int64_t rb = p.a_kblock == 0 ? p.lda * 2 : 64;
      d_off[j] = arow >= 0 ? static_cast<uint32_t>(arow * rb) + c * 16u : kOutOfRange;
    } else {
      const int n = (q - ACH) / kGgBKC;
      const int c = ((q - ACH) % kGgBKC) ^ gg_swz(n);
      // row-major B: stage 0 of row col0 + n; banded B: the tile's band,
      // its first block, row n
      d_off[j] = p.b_bands ? static_cast<uint32_t>((int64_t)t.col0 * p.K * 2 + n * 64) + c * 16u
                           : static_cast<uint32_t>((int64_t)(t.col0 + n) * p.ldb * 2) + c * 16u;
    }
  }
  // stage kt -> ring buffer kt % kGgNS; stages past the end load zeros
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)gg_ring)));
  // bytes between K stages: 32 elements of a row, or (blocked A) a block
  const uint32_t a_step = p.a_kblock == 0 ? kGgBK * 2u : static_cast<uint32_t>(p.a_kblock) * 64u;
  const uint32_t b_step = p.b_bands ? kGgBN * kGgBK * 2u : kGgBK * 2u;
  auto issue_part = [&](int kt, int j0, int j1) {
    const uint32_t s_ = ring_lds + static_cast<uint32_t>((kt % kGgNS) * kGgStage * 16);
    const uint32_t kb = static_cast<uint32_t>(kt) * b_step;
    const uint32_t ka = static_cast<uint32_t>(kt) * a_step;
    const bool live = kt < nk;
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const bool is_a = (kGgNW * j + wave) * 64 < ACH;  // wave-uniform
      gg_dma(is_a ? a_rsrc : b_rsrc, s_ + static_cast<uint32_t>((kGgNW * j + wave) * 64 * 16),
             live ? d_off[j] + (is_a ? ka : kb) : kOutOfRange);
    }
  };
  auto issue = [&](int kt) { issue_part(kt, 0, NDMA); };
  // the loads of stage kt + 3: NA of them in k-step 0, NB in k-step 1.  FC1
  // (gathered rows, K = l) measured 3 % faster with the loads split over
  // both k-steps, FC2 (K = m) 3 % slower; so only the gathering instance
  // splits them.
  constexpr int NA = GATHER ? (NDMA + 1) / 2 : NDMA, NB = NDMA - NA;

  // fragments of k-step ks (two chunks of K per 32x32x16 MFMA) of stage kt
  const int frow = lane & 31, fchk = lane >> 5;
  u32x4 fa[2][MI], fb[2][kGgNJ];
#define GG_FRAGS(kt, ks, f)                                                      \
  do {                                                                           \
    const u32x4* s_ = gg_ring + ((kt) % kGgNS) * kGgStage;                       \
    const int c_ = 2 * (ks) + fchk;                                              \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) {                             \
      const int r_ = wm * WM + i * 32 + frow;                                    \
      fa[f][i] = s_[r_ * kGgBKC + (c_ ^ gg_swz(r_))];                            \
    }                                                                            \
    _Pragma("unroll") for (int j = 0; j < kGgNJ; ++j) {                          \
      const int n_ = wn * kGgWCols + j * 32 + frow;                              \
      fb[f][j] = s_[ACH + n_ * kGgBKC + (c_ ^ gg_swz(n_))];                      \
    }                                                                            \
  } while (0)
#define GG_MMA(f)                                                                \
  do {                                                                           \
    _Pragma("unroll") for (int i = 0; i < MI; ++i)                               \
    _Pragma("unroll") for (int j = 0; j < kGgNJ; ++j)                            \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                       \
          __builtin_bit_cast(bf16x8_t, fb[f][j]), __builtin_bit_cast(bf16x8_t, fa[f][i]), \
          acc[i][j], 0, 0, 0);                                                   \
  } while (0)
  // a k-step: its MFMAs with the next k-step's fragment reads in front
  // (one read, one MFMA), then its share of the next stage's loads
#define GG_SCHED(loads)                                                          \
  do {                                                                           \
    _Pragma("unroll") for (int q_ = 0; q_ < MI + kGgNJ; ++q_) {                  \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                         \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         \
    }                                                                            \
    if ((loads) > 0) {                                                           \
      _Pragma("unroll") for (int q_ = 0; q_ < (loads); ++q_) {                   \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       \
      }                                                                          \
    }                                                                            \
    __builtin_amdgcn_sched_group_barrier(0x008, kGgNJ * MI, 0);                  \
  } while (0)

#pragma unroll
  for (int s = 0; s < kGgNS - 1; ++s) issue(s);
  // the next tile's source rows, behind this tile's first stages: the waits
  // below then also cover them (one load more than a stage may stay in
  // flight at the first wait), and they have landed after k-step 0
  if (GATHER && next_row0 >= 0 && wave < kGgBM / 64)
    gg_fetch_rows(p, total_rows, next_row0, buf ^ 1, wave, lane);
  wait_vmcnt_lgkm0<(kGgNS - 2) * NDMA>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  GG_FRAGS(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    // k-step 0: fragments of k-step 1 in front, then the first NA loads of
    // stage kt + 3 into the buffer stage kt - 1 used (every wave finished
    // reading it before the last barrier)
    GG_FRAGS(kt, 1, 1);
    issue_part(kt + kGgNS - 1, 0, NA);
    GG_MMA(0);
    GG_SCHED(NA);
    // k-step 0's MFMAs stay in front of the wait (the scheduler would move
    // some of them past the barrier, and the wave would wait with the MFMA
    // pipe idle)
    __builtin_amdgcn_sched_barrier(0);
    // stage kt + 1 landed (this thread's loads, issued before stage kt + 2's
    // and the first NA of stage kt + 3, which may stay in flight; the
    // barrier makes it everyone's), this wave's fragment reads done
    wait_vmcnt_lgkm0<(kGgNS - 3) * NDMA + NA>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 1: stage kt + 1's first fragments in front, then the rest of
    // stage kt + 3's loads (into the same buffer, read by no wave since the
    // last barrier)
    GG_FRAGS(kt + 1, 0, 0);
    issue_part(kt + kGgNS - 1, NA, NDMA);
    GG_MMA(1);
    GG_SCHED(NB);
  }
#undef GG_SCHED
#undef GG_MMA
#undef GG_FRAGS
  // the ring is reused by the next tile: every load and read done
  wait_vmcnt_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue, one 32-row block row at a time: lane holds row frow of
  // each block, columns 8 g + 4 (lane / 32) + 0..3 in accumulator elements
  // 4 g .. 4 g + 3; they go to the wave's staging area (activated, in bf16)
  // and leave as 16-byte chunks, 8 lanes per 128-byte row segment (64
  // bytes with SwiGLU, whose output is half as wide).  LDS operations of one
  // wave complete in order, so the reads see the writes.  The stores are
  // buffer stores whose range ends at the tile's last row: those of rows
  // past it are dropped by the range check, without a per-store test.
  constexpr int OW = ACT == kActSwiGlu ? kGgWCols / 2 : kGgWCols;  // output columns of a wave
  constexpr int CPR = OW / 8;                        // 16-byte chunks per staged row
  constexpr int RPS = 64 / CPR;                      // rows per wave store
  uint16_t* stg = reinterpret_cast<uint16_t*>(gg_ring + (kGgNS - 1) * kGgStage) + wave * 32 * kGgOutLd;
  const int ocol0 = (ACT == kActSwiGlu ? t.col0 / 2 : t.col0) + wn * OW;
  const int srow = lane / CPR, sch = lane % CPR;     // this lane's staged row / chunk
  // row-major C: a resource whose range ends at the tile's last row, rows
  // past it dropped by the range check; blocked C (chunk in block
  // (ocol0 + 8 sch) / 32): the whole array, rows past the tile offset out
  // of range per lane
  const bool cblk = p.c_kblock > 0;
  const uint32_t ldc2 = cblk ? 64u : static_cast<uint32_t>(p.ldc) * 2;
  const int out_cols = ACT == kActSwiGlu ? p.N / 2 : p.N;
  const BufRsrc c_rsrc = make_rsrc(
      p.C, cblk ? static_cast<uint64_t>(p.c_kblock) * out_cols * 2
                : static_cast<uint64_t>(t.row0 + t.rows) * ldc2);
  const int ccol = ocol0 + sch * 8;
  const uint32_t c_off =
      cblk ? static_cast<uint32_t>((ccol >> 5) * p.c_kblock + t.row0 + wm * WM + srow) * 64u +
                 static_cast<uint32_t>(ccol & 31) * 2u
           : static_cast<uint32_t>(t.row0 + wm * WM + srow) * ldc2 + static_cast<uint32_t>(ccol) * 2;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < kGgNJ; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = j * 32 + 8 * g4 + 4 * fchk;   // column within the wave's 64
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = apply_act<ACT>(acc[i][j][4 * g4 + e]);
        if constexpr (ACT == kActSwiGlu) {
          *reinterpret_cast<uint32_t*>(stg + frow * kGgOutLd + c / 2) =
              pack_bf16x2(swiglu(v[0], v[1]), swiglu(v[2], v[3]));
        } else {
          *reinterpret_cast<uint2*>(stg + frow * kGgOutLd + c) =
              uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
#pragma unroll
    for (int u = 0; u < 32 / RPS; ++u) {
      const u32x4 val =
          *reinterpret_cast<const u32x4*>(stg + (u * RPS + srow) * kGgOutLd + sch * 8);
      const int r = wm * WM + i * 32 + u * RPS + srow;   // row within the tile
      const uint32_t off = c_off + static_cast<uint32_t>(i * 32 + u * RPS) * ldc2;
      // non-temporal: the output is read again only by the next kernel
      // (FC1: 2 % faster)
      __builtin_amdgcn_raw_buffer_store_b128(val, c_rsrc, !cblk || r < t.rows ? off : kOutOfRange,
                                             0, kCpolNonTemporal);
      // dense: the optional blocked copy (C2, M rows per block), rows past
      // the tile offset out of range per lane
      if constexpr (DENSE) {
        if (p.C2 != nullptr) {
          const BufRsrc c2_rsrc = make_rsrc(p.C2, static_cast<uint64_t>(p.M) * p.N * 2);
          const uint32_t off2 =
              static_cast<uint32_t>((ccol >> 5) * p.M + t.row0 + r) * 64u +
              static_cast<uint32_t>(ccol & 31) * 2u;
          __builtin_amdgcn_raw_buffer_store_b128(val, c2_rsrc, r < t.rows ? off2 : kOutOfRange, 0, 0);
        }
      }
    }
  }
}

// DENSE: one group of p.M rows, no g_off (a dense GEMM on the same tiles;
// its own instance, so that profiles tell it from the expert GEMMs)
template <int ACT, bool GATHER, bool DENSE>
__global__ __launch_bounds__(kGgNT, 1) void gemm_grouped_kernel(GemmArgs p) {
  __shared__ int s_pre[kGgMaxG + 1];         // items before expert e
  __shared__ int s_off[kGgMaxG + 1];         // g_off
  __shared__ int s_wsum[kGgNW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int ncol = p.N / kGgBN;

  // ---- items of each expert: ceil(rows / 256) row tiles x ncol column
  // tiles; exclusive prefix over the experts (8 per thread)
  int v[8], sum = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = tid * 8 + u;
    v[u] = 0;
    if (e < G) {
      const int o0 = DENSE ? 0 : p.g_off[e], o1 = DENSE ? p.M : p.g_off[e + 1];
      s_off[e] = o0;
      if (e == G - 1) s_off[G] = o1;
      v[u] = (o1 - o0 + kGgBM - 1) / kGgBM * ncol;
    }
    sum += v[u];
  }
  int inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  int ex = inc - sum, total = 0;
  for (int w = 0; w < kGgNW; ++w) {
    if (w < wave) ex += s_wsum[w];
    total += s_wsum[w];
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = tid * 8 + u;
    if (e < G) s_pre[e] = ex;
    ex += v[u];
  }
  if (tid == 0) s_pre[G] = total;
  __syncthreads();

  // ---- this workgroup's items: its XCD's contiguous range, strided by the
  // XCD's workgroup count
  const int nx = gridDim.x / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd, j = blockIdx.x / kNumXcd;
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int i1 = min(total, (xcd + 1) * per);
  const int total_rows = __builtin_amdgcn_readfirstlane(s_off[G]);
  // the expert of an item: the last one whose first item is <= item (items
  // only increase along a workgroup's walk: the expert only advances; the
  // sentinel s_pre[G] = total ends the scan)
  auto advance = [&](int g, int item) {
    while (s_pre[g + 1] <= item) ++g;
    return __builtin_amdgcn_readfirstlane(g);
  };
  // the tile of an item of expert g; wave-uniform values, kept in scalar
  // registers
  auto tile_of = [&](int g, int item) {
    const int li = item - __builtin_amdgcn_readfirstlane(s_pre[g]);
    const int rt = li / ncol;
    GgTile t;
    t.g = g;
    t.row0 = __builtin_amdgcn_readfirstlane(s_off[g]) + rt * kGgBM;
    t.rows = min(kGgBM, __builtin_amdgcn_readfirstlane(s_off[g + 1]) - t.row0);
    t.col0 = (li - rt * ncol) * kGgBN;
    return t;
  };
  int item = xcd * per + j;
  if (item >= i1) return;
  int g = 0;  // the first item's expert: a binary search
  for (int step = kGgMaxG / 2; step > 0; step >>= 1)
    if (g + step < G && s_pre[g + step] <= item) g += step;
  g = __builtin_amdgcn_readfirstlane(g);
  if (GATHER) {  // the first tile's source rows
    if (wave < kGgBM / 64) gg_fetch_rows(p, total_rows, tile_of(g, item).row0, 0, wave, lane);
    wait_vmcnt_lgkm0<0>();
    __syncthreads();
  }
  GgAcc acc;
  for (int buf = 0; item < i1; item += nx, buf ^= 1) {
    const GgTile t = tile_of(g, item);
    const bool more = item + nx < i1;
    if (more) g = advance(g, item + nx);
    const int next_row0 = GATHER && more ? tile_of(g, item + nx).row0 : -1;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < kGgNJ; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
    if (t.rows > 128) gg_tile<4, ACT, GATHER, DENSE>(p, t, wave, lane, acc, buf, next_row0, total_rows);
    else if (t.rows > 64) gg_tile<2, ACT, GATHER, DENSE>(p, t, wave, lane, acc, buf, next_row0, total_rows);
    else gg_tile<1, ACT, GATHER, DENSE>(p, t, wave, lane, acc, buf, next_row0, total_rows);
  }
}

}  // namespace

bool gemm_grouped_fits(int N, int K, int G) {
  return N > 0 && K > 0 && N % kGgBN == 0 && K % kGgBK == 0 && G >= 1 && G <= kGgMaxG;
}

namespace {

// One 16-byte chunk per thread, grid-stride: source chunk i of the
// row-major matrices is row n = (i / cpr) % N of matrix g, chunk kc = i %
// cpr (cpr chunks per row); it goes to band n / R, 64-byte block kc / 4,
// row n % R, chunk kc % 4 of that block.
__global__ __launch_bounds__(256) void pack_bands_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t chunks,
                                                         int N, int cpr, int R) {
  const int64_t per_g = static_cast<int64_t>(N) * cpr;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < chunks;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t g = i / per_g, rem = i % per_g;
    const int64_t n = rem / cpr, kc = rem % cpr;
    const int64_t o = g * per_g + ((n / R) * (cpr / 4) + kc / 4) * (4 * R) + (n % R) * 4 + kc % 4;
    dst[o] = src[i];
  }
}

}  // namespace

hipError_t launch_pack_bands(const void* src, void* dst, int G, int N, int row_bytes, int band_rows,
                             hipStream_t s) {
  if (!src || !dst || G < 1 || N < 1 || row_bytes < 64 || band_rows < 1 || N % band_rows ||
      row_bytes % 64 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u))
    return hipErrorInvalidValue;
  const int64_t chunks = static_cast<int64_t>(G) * N * (row_bytes / 16);
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 65536);
  pack_bands_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), chunks, N, row_bytes / 16,
      band_rows);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t s) {
  if (!gemm_grouped_fits(a.N, a.K, a.G) || a.b_scale || a.B2 || a.R || a.b_mx || a.a_nrows <= 0 ||
      a.max_rows <= 0)
    return hipErrorInvalidValue;
  // dense: one group of M rows, A not gathered, every row of A and C there
  if (a.g_off == nullptr &&
      (a.G != 1 || a.M <= 0 || a.a_rows || a.a_nrows < a.M || a.max_rows < a.M))
    return hipErrorInvalidValue;
  // the blocked copy: dense, no activation, whole 32-column blocks, 32-bit offsets
  if (a.C2 && (a.g_off != nullptr || a.act != kActNone || a.N % 32 ||
               (uint64_t)a.M * a.N * 2 >= (1ull << 31) ||
               (reinterpret_cast<uintptr_t>(a.C2) & 15u)))
    return hipErrorInvalidValue;
  const int out_cols = a.act == kActSwiGlu ? a.N / 2 : a.N;
  if (a.c_kblock == 0 && a.ldc < out_cols) return hipErrorInvalidValue;
  // blocked A: not gathered, every row of A in the blocks; blocked C: every
  // row the launch writes in the blocks, whole 32-column blocks
  if (a.a_kblock < 0 || a.c_kblock < 0 || (a.a_kblock > 0 && a.a_kblock < a.a_nrows) ||
      (a.c_kblock > 0 && (a.c_kblock < a.max_rows || out_cols % 32)) ||
      (a.b_bands && a.ldb != a.K))
    return hipErrorInvalidValue;
  // 32-bit buffer offsets: A, one expert's B, C (max_rows bounds its rows)
  const uint64_t a_bytes = a.a_kblock ? (uint64_t)a.a_kblock * a.K * 2 : (uint64_t)a.a_nrows * a.lda * 2;
  const uint64_t c_bytes = a.c_kblock ? (uint64_t)a.c_kblock * out_cols * 2 : (uint64_t)a.max_rows * a.ldc * 2;
  if (a_bytes >= (1ull << 31) || (uint64_t)a.N * a.ldb * 2 >= (1ull << 31) || c_bytes >= (1ull << 31))
    return hipErrorInvalidValue;
  const int grid = (device_compute_units() + kNumXcd - 1) / kNumXcd * kNumXcd;
  const bool g = a.a_rows != nullptr;
  if (a.g_off == nullptr) {
    if (a.act != kActNone) return hipErrorInvalidValue;
    gemm_grouped_kernel<kActNone, false, true><<<grid, kGgNT, 0, s>>>(a);
  } else if (a.act == kActSqRelu) {
    if (g) gemm_grouped_kernel<kActSqRelu, true, false><<<grid, kGgNT, 0, s>>>(a);
    else gemm_grouped_kernel<kActSqRelu, false, false><<<grid, kGgNT, 0, s>>>(a);
  } else if (a.act == kActSwiGlu) {
    if (g) gemm_grouped_kernel<kActSwiGlu, true, false><<<grid, kGgNT, 0, s>>>(a);
    else gemm_grouped_kernel<kActSwiGlu, false, false><<<grid, kGgNT, 0, s>>>(a);
  } else {
    if (g) gemm_grouped_kernel<kActNone, true, false><<<grid, kGgNT, 0, s>>>(a);
    else gemm_grouped_kernel<kActNone, false, false><<<grid, kGgNT, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace lmoe
