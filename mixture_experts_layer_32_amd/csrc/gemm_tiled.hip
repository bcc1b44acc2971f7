// LDS-tiled MFMA GEMM, dense or grouped by expert, for gfx950.
//
// C[r][n] = act(sum_k A[arow(r)][k] * B[g][n][k])  (+ R[r][n], dense)
//
// Used for the two projections (W_down: u = x W_down^T, W_up: out = v W_up^T),
// the router logits (fp32 output) and, when experts receive many tokens, the
// grouped latent expert GEMMs (FC1 gathers token rows through token_of).
//
// Block tile BM x BN computed by WGM x WGN waves, each wave a (BM / WGM) x
// (BN / WGN) sub-tile of 16x16 or 32x32 MFMA blocks; a larger wave sub-tile
// reuses every LDS fragment for more MFMAs, and a larger block tile needs
// fewer operand bytes per flop (the main loop is bound by how many bytes
// are in flight against the latency of the loads).
// K advances in stages of BKC 16-byte chunks per row.
//
// Operands move from global memory straight into an LDS ring of NSTAGE
// stage buffers with buffer loads in LDS mode (no register staging): while
// stage kt is multiplied, stages kt+1 .. kt+NSTAGE-1 are in flight.  Every
// thread issues the same number of loads per stage (out-of-range offsets
// write zeros without touching memory: padding rows, K tails, stages past the
// end), so "stage kt+1 has landed" is an exact vmcnt wait, followed by one
// barrier per stage.  MFMA fragments are double-buffered in registers: the
// fragment reads of the next k-step overlap the MFMAs of the current one,
// also across the stage barrier.
//
// LDS rows hold BKC chunks; logical chunk c of row r sits at position
// c ^ swz(r) (swz(r) = (r >> 1) & 7 for 8-chunk rows, (r >> 2) & 3 for 4-chunk
// rows), so the 16 lanes reading one fragment column of 16 consecutive rows
// touch 16 distinct 16-byte bank groups.  The output tile leaves through LDS
// (rows padded by 16 bytes against bank conflicts) as 16-byte row chunks.
// An optional fp32 residual R (the shared experts' sum, added to W_up's
// output) joins the accumulators before the one rounding to the output type.
//
// Dense problems with too few tiles to fill the device split K: every split
// writes an fp32 partial tile and a reduction kernel adds the partials in a
// fixed order (deterministic), then activates and converts.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

template <int BM_, int BN_, int WGM_, int WGN_, int BKC_, int NSTAGE_, int OCC_ = 1>
struct TileCfg {
  static constexpr int OCC = OCC_;               // workgroups per compute unit to fit
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WGM = WGM_, WGN = WGN_;  // waves along M and N
  static constexpr int NW = WGM_ * WGN_;         // waves per workgroup
  static constexpr int NT = 64 * NW;             // threads per workgroup
  static constexpr int BKC = BKC_;               // 16-byte chunks per row per stage
  static constexpr int NSTAGE = NSTAGE_;
};
// tile configurations (index = the `tile` argument of launch_gemm_tiled)
using Tile128 = TileCfg<128, 128, 2, 2, 8, 2, 2>;  // 0: 4 waves of 64x64
using Tile64 = TileCfg<64, 64, 2, 2, 8, 4>;                 // 1: 4 waves of 32x32
using Tile256 = TileCfg<256, 256, 2, 4, 4, 4>;              // 2: 8 waves of 128x64 (bf16 output only)
using Tile128x256 = TileCfg<128, 256, 2, 2, 4, 3, 2>;  // 3: 4 waves of 64x128

template <int BKC>
__device__ __forceinline__ int lds_swz(int r) {
  return BKC == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// four consecutive output values to LDS in one store (8 or 16 bytes, aligned)
template <typename TOut>
__device__ __forceinline__ void store4(TOut* p, const float (&v)[4]);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const float (&v)[4]) {
  uint2 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = w;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&v)[4]) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
}
// two consecutive output values (4 or 8 bytes, aligned)
template <typename TOut>
__device__ __forceinline__ void store2(TOut* p, float a, float b);
template <>
__device__ __forceinline__ void store2<uint16_t>(uint16_t* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}
template <>
__device__ __forceinline__ void store2<float>(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = float2{a, b};
}

template <typename Mma, typename TA, typename TOut, typename Cfg, int ACT>
__global__ __launch_bounds__(Cfg::NT, Cfg::OCC) void gemm_tiled_kernel(GemmArgs p, int splits, float* partial) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BKC = Cfg::BKC, NSTAGE = Cfg::NSTAGE;
  constexpr int EPC = 16 / sizeof(TA);       // A elements per 16-byte chunk
  constexpr int BKE = BKC * EPC;             // elements of K per stage
  using TB = TA;                             // B is the A type
  constexpr int EPCB = EPC;                  // B elements per chunk
  constexpr int BKCB = BKC;                  // B chunks per row per stage
  constexpr int KS = BKC / Mma::CPS;         // MFMA k-steps per stage
  constexpr int WM = BM / Cfg::WGM, WN = BN / Cfg::WGN;
  constexpr int BLK = Mma::BLK, NV = Mma::NV;
  constexpr int MI = WM / BLK, NI = WN / BLK;
  static_assert(WM % BLK == 0 && WN % BLK == 0, "wave tile must hold whole MFMA blocks");
  constexpr int ACH = BM * BKC;              // A chunks per stage (first in the buffer)
  constexpr int STAGE = ACH + BN * BKCB;     // chunks per LDS stage buffer
  constexpr int NW = Cfg::NW, NT = Cfg::NT;
  constexpr int NDMA = STAGE / NT;           // LDS-mode loads per thread per stage
  constexpr int OPAD = 16 / sizeof(TOut);    // output tile row padding (elements)
  constexpr bool PARTIAL_OK = BM * BN <= 128 * 128;
  constexpr size_t RING = size_t(NSTAGE) * STAGE * 16;
  constexpr size_t OUT_T = size_t(BM) * (BN + OPAD) * sizeof(TOut);
  constexpr size_t OUT_P = PARTIAL_OK ? size_t(BM) * (BN + 4) * 4 : 0;
  static_assert(STAGE % NT == 0 && ACH % 64 == 0, "stage must split into wave loads");
  static_assert(BKC == 4 || BKC == 8, "stage row = 64 or 128 bytes");
  __shared__ u32x4 smem[cmax(RING, cmax(OUT_T, OUT_P)) / 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform across the wave: say so, so that values
  // derived from it (buffer resource choice, LDS bases) live in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_tiles = (p.N + BN - 1) / BN;

  // ---- which tile (and which K split)
  int g = 0, row0, rows, col0, kz = 0;
  if (p.g_off == nullptr) {
    const int mn = ((p.M + BM - 1) / BM) * n_tiles;
    const int item = xcd_contiguous_item(blockIdx.x, gridDim.x, mn * splits);
    if (item < 0) return;
    kz = item / mn;                      // splits outermost: neighbours share A rows
    const int t = item % mn;
    row0 = (t / n_tiles) * BM;
    col0 = (t % n_tiles) * BN;
    rows = min(BM, p.M - row0);
  } else {
    const int total = p.g_tiles[p.G] * n_tiles;
    const int item = xcd_contiguous_item(blockIdx.x, gridDim.x, total);
    if (item < 0) return;
    const int mg = item / n_tiles;
    col0 = (item % n_tiles) * BN;
    int lo = 0, hi = p.G - 1;  // last group whose first tile is <= mg
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.g_tiles[mid] <= mg) lo = mid; else hi = mid - 1;
    }
    // wave-uniform values (the buffer resources built from them must sit in
    // scalar registers)
    g = __builtin_amdgcn_readfirstlane(lo);
    const int gs = __builtin_amdgcn_readfirstlane(p.g_off[g]);
    const int ge = __builtin_amdgcn_readfirstlane(p.g_off[g + 1]);
    row0 = gs + (mg - __builtin_amdgcn_readfirstlane(p.g_tiles[g])) * BM;
    rows = min(BM, ge - row0);
  }
  // K range of this split, in whole stages
  const int nk_all = (p.K + BKE - 1) / BKE;
  const int per = (nk_all + splits - 1) / splits;
  const int kt0 = kz * per;
  const int nk = max(0, min(nk_all, kt0 + per) - kt0);
  const int k_end = min(p.K, (kt0 + nk) * BKE);

  const TA* A = static_cast<const TA*>(p.A);
  const TB* B = static_cast<const TB*>(p.B) + (int64_t)g * p.b_gstride;
  // columns from the second weight matrix: this tile's rows of B are
  // bn0 .. of B2 (the host keeps N0 a multiple of BN)
  int bn0 = 0, bN = p.N;
  if (p.B2) {
    if (col0 >= p.N0) {
      B = static_cast<const TB*>(p.B2);
      bn0 = p.N0;
      bN = p.N - p.N0;
    } else {
      bN = p.N0;
    }
  }
  const uint64_t a_rows_total = p.g_off ? (uint64_t)p.a_nrows : (uint64_t)p.M;
  const BufRsrc a_rsrc = make_rsrc(A, a_rows_total * p.lda * sizeof(TA));
  const BufRsrc b_rsrc = make_rsrc(B, (uint64_t)bN * p.ldb * sizeof(TB));

  // ---- LDS-mode staging.  Stage buffer position q (16-byte chunks): A row
  // q / BKC for q < ACH, else B row (q - ACH) / BKCB; within a row, logical
  // chunk c sits at position c ^ swz(row).  Load j of wave w fills positions
  // (NW j + w) * 64 + lane, so each lane's row and chunk are fixed; per stage
  // only the K offset changes.
  uint32_t d_off[NDMA];  // byte offset in A or B of this lane's chunk at K stage 0
  int d_k[NDMA];         // its first K element
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int q = (NW * j + wave) * 64 + lane;
    if (q < ACH) {
      const int r = q / BKC;
      const int c = (q % BKC) ^ lds_swz<BKC>(r);
      d_k[j] = c * EPC;
      int64_t arow = -1;
      if (r < rows) arow = p.a_rows ? p.a_rows[row0 + r] : row0 + r;
      d_off[j] = arow >= 0 ? static_cast<uint32_t>(arow * p.lda * sizeof(TA)) + c * 16u : kOutOfRange;
    } else {
      const int r = (q - ACH) / BKCB;
      const int c = ((q - ACH) % BKCB) ^ lds_swz<BKCB>(r);
      d_k[j] = c * EPCB;
      const int n = col0 - bn0 + r;
      d_off[j] = n < bN ? static_cast<uint32_t>((int64_t)n * p.ldb * sizeof(TB)) + c * 16u
                        : kOutOfRange;
    }
  }
  // stage kt -> ring buffer kt % NSTAGE, always NDMA loads per thread
  auto issue_stage = [&](int kt) {
    u32x4* s_ = smem + (kt % NSTAGE) * STAGE;
    const int kb = (kt0 + kt) * BKE;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const bool in_ = kt < nk && kb + d_k[j] < k_end && d_off[j] != kOutOfRange;
      const bool is_a = (NW * j + wave) * 64 < ACH;  // wave-uniform
      const uint32_t kbytes = static_cast<uint32_t>(kb) * (is_a ? sizeof(TA) : sizeof(TB));
      buffer_load_chunk_lds(is_a ? a_rsrc : b_rsrc, s_ + (NW * j + wave) * 64,
                            in_ ? d_off[j] + kbytes : kOutOfRange);
    }
  };

  typename Mma::Acc acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[i][j][v] = 0.f;

  const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
  // MFMA operand fragments of one k-step (CPS chunks of K, one MFMA per
  // block pair): logical chunk CPS ks + frag_chunk(lane) of fragment row
  // frag_row(lane), for this wave's m-blocks (A) and n-blocks (B)
  const int frow = Mma::frag_row(lane);
  const int fchk = Mma::frag_chunk(lane);
  u32x4 fa[2][MI], fb[2][NI];
#define LMOE_FRAGS(kt, ks, f)                                                           \
  do {                                                                                  \
    const u32x4* s_ = smem + ((kt) % NSTAGE) * STAGE;                                   \
    const int c_ = (ks) * Mma::CPS + fchk;                                              \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                    \
      const int r_ = wm * WM + i * BLK + frow;                                          \
      fa[f][i] = s_[r_ * BKC + (c_ ^ lds_swz<BKC>(r_))];                                \
    }                                                                                   \
    _Pragma("unroll") for (int j = 0; j < NI; ++j) {                                    \
      const int r_ = wn * WN + j * BLK + frow;                                          \
      fb[f][j] = s_[ACH + r_ * BKCB + (c_ ^ lds_swz<BKCB>(r_))];                        \
    }                                                                                   \
  } while (0)
#define LMOE_MMA(f)                                                                     \
  do {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < MI; ++i)                                      \
    _Pragma("unroll") for (int j = 0; j < NI; ++j) Mma::mma(acc[i][j], fb[f][j], fa[f][i]); \
  } while (0)
  // after each LDS fragment read, a share of the MFMAs already possible
#define LMOE_INTERLEAVE()                                                               \
  do {                                                                                  \
    _Pragma("unroll") for (int q_ = 0; q_ < MI + NI; ++q_) {                            \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                \
      __builtin_amdgcn_sched_group_barrier(0x008, (MI * NI + MI + NI - 1) / (MI + NI), 0); \
    }                                                                                   \
  } while (0)
  // Stage kt whose k-step 0 fragments are in register set P: issue the loads
  // of stage kt+NSTAGE-1 (into the buffer stage kt-1 used, which every wave
  // finished reading before the previous barrier); run the k-steps, reading
  // the next k-step's fragments during each; wait until this thread's loads
  // of stage kt+1 have landed and its fragment reads are done, barrier (then
  // every thread's stage kt+1 is in LDS); read stage kt+1's k-step 0
  // fragments during the last k-step's MFMAs.
#define LMOE_STAGE(kt, P)                                                               \
  do {                                                                                  \
    issue_stage((kt) + NSTAGE - 1);                                                     \
    _Pragma("unroll") for (int ks = 0; ks + 1 < KS; ++ks) {                             \
      LMOE_FRAGS(kt, ks + 1, ((P) + ks + 1) & 1);                                       \
      LMOE_MMA(((P) + ks) & 1);                                                         \
      LMOE_INTERLEAVE();                                                                \
    }                                                                                   \
    wait_vmcnt_lgkm0<(NSTAGE - 2) * NDMA>();                                            \
    __builtin_amdgcn_s_barrier();                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    LMOE_FRAGS((kt) + 1, 0, ((P) + KS) & 1);                                            \
    LMOE_MMA(((P) + KS - 1) & 1);                                                       \
    LMOE_INTERLEAVE();                                                                  \
  } while (0)

#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) issue_stage(s);
  wait_vmcnt_lgkm0<(NSTAGE - 2) * NDMA>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  LMOE_FRAGS(0, 0, 0);
  // with an even number of k-steps per stage every stage starts from
  // register set 0: one stage per iteration, so the accumulators keep their
  // registers across iterations
  static_assert(KS % 2 == 0, "stages must hold an even number of MFMA k-steps");
  for (int kt = 0; kt < nk; ++kt) LMOE_STAGE(kt, 0);
#undef LMOE_STAGE
#undef LMOE_INTERLEAVE
#undef LMOE_MMA
#undef LMOE_FRAGS
  // loads of stages past the last one still target the ring: let them land
  // before the buffers are reused for the output tile
  wait_vmcnt_lgkm0<0>();
  __syncthreads();

  // ---- epilogue through LDS: direct output (scale, act, convert) or fp32 partial
  if (partial == nullptr) {
    // SwiGLU: column pairs (up, gate) become one output column, the tile is
    // BN / 2 wide
    constexpr bool GLU = ACT == kActSwiGlu;
    constexpr int BNO = GLU ? BN / 2 : BN;
    constexpr int LDT = BNO + OPAD;  // LDS tile row stride (elements)
    static_assert(OUT_T <= sizeof(smem), "output tile must fit LDS");
    TOut* Ct = reinterpret_cast<TOut*>(smem);
    // blocks are held transposed (B fragment first in the MFMA): each group of
    // 4 accumulator elements is 4 consecutive columns of one row, written to
    // LDS as one 8-byte (bf16) or 16-byte (fp32) store
    const int trow = Mma::t_row(lane);
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int g4 = 0; g4 < NV / 4; ++g4) {
        const int colt = wn * WN + j * BLK + Mma::t_col(lane, g4);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          float val[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = apply_act<ACT>(acc[i][j][4 * g4 + e]);
          if constexpr (GLU) {
            store2<TOut>(Ct + (wm * WM + i * BLK + trow) * LDT + colt / 2, swiglu(val[0], val[1]),
                         swiglu(val[2], val[3]));
            continue;
          }
          // residual (dense, N % 4 == 0: the 4 columns are in or out together)
          const int lr = wm * WM + i * BLK + trow;
          if (p.R != nullptr && lr < rows && col0 + colt < p.N) {
            const f32x4_t r4 =
                *reinterpret_cast<const f32x4_t*>(p.R + (int64_t)(row0 + lr) * p.ldr + col0 + colt);
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] += r4[e];
          }
          store4<TOut>(Ct + (wm * WM + i * BLK + trow) * LDT + colt, val);
        }
      }
    __syncthreads();
    constexpr int EPO = 16 / sizeof(TOut);
    constexpr int CPR = BNO / EPO;
    TOut* C = static_cast<TOut*>(p.C);
    const int n_out = GLU ? p.N / 2 : p.N;
    const int col_out = GLU ? col0 / 2 : col0;
    // whole 16-byte chunks where the row stride keeps them aligned and the
    // chunk lies inside N; element stores otherwise (e.g. N = expert count)
    const bool aligned = (p.ldc % EPO) == 0;
    for (int q = tid; q < rows * CPR; q += NT) {
      const int r = q / CPR, ch = q % CPR;
      const int col = col_out + ch * EPO;
      TOut* dst = C + (int64_t)(row0 + r) * p.ldc + col;
      const TOut* src = Ct + r * LDT + ch * EPO;
      if (aligned && col + EPO <= n_out) {
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
      } else {
        for (int e = 0; e < EPO && col + e < n_out; ++e) dst[e] = src[e];
      }
    }
  } else if constexpr (PARTIAL_OK) {
    constexpr int LDP = BN + 4;
    float* Pt = reinterpret_cast<float*>(smem);
    const int trow = Mma::t_row(lane);
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int g4 = 0; g4 < NV / 4; ++g4)
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          float val[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = acc[i][j][4 * g4 + e];
          store4<float>(Pt + (wm * WM + i * BLK + trow) * LDP + wn * WN + j * BLK +
                            Mma::t_col(lane, g4), val);
        }
    __syncthreads();
    constexpr int CPR = BN / 4;
    float* P = partial + (int64_t)kz * p.M * p.N;
    for (int q = tid; q < rows * CPR; q += NT) {
      const int r = q / CPR, ch = q % CPR;
      const int col = col0 + ch * 4;
      if (col < p.N)
        *reinterpret_cast<u32x4*>(P + (int64_t)(row0 + r) * p.N + col) =
            *reinterpret_cast<const u32x4*>(Pt + r * LDP + ch * 4);
    }
  }
}

// C[r][c] = act(sum_s P[s][r][c]) (+ R[r][c]), splits added in order.
template <typename TOut, int ACT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int splits,
                                                            int M, int N,
                                                            const float* __restrict__ R, int64_t ldr,
                                                            TOut* __restrict__ C, int64_t ldc) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4 columns per thread
  const int64_t total = (int64_t)M * (N / 4);
  if (q >= total) return;
  const int r = static_cast<int>(q / (N / 4));
  const int c = static_cast<int>(q % (N / 4)) * 4;
  const int64_t mn = (int64_t)M * N;
  f32x4_t s = *reinterpret_cast<const f32x4_t*>(P + (int64_t)r * N + c);
  for (int z = 1; z < splits; ++z) s += *reinterpret_cast<const f32x4_t*>(P + z * mn + (int64_t)r * N + c);
  if constexpr (ACT == kActSwiGlu) {  // columns (c, c+1), (c+2, c+3) -> c/2, c/2 + 1
    store_elem<TOut>(C + (int64_t)r * ldc + c / 2, swiglu(s[0], s[1]));
    store_elem<TOut>(C + (int64_t)r * ldc + c / 2 + 1, swiglu(s[2], s[3]));
    return;
  }
  f32x4_t res = {0.f, 0.f, 0.f, 0.f};
  if (R != nullptr) res = *reinterpret_cast<const f32x4_t*>(R + (int64_t)r * ldr + c);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float val = apply_act<ACT>(s[v]);
    if (R != nullptr) val += res[v];
    store_elem<TOut>(C + (int64_t)r * ldc + c + v, val);
  }
}

template <typename Mma, typename TA, typename TOut, typename Cfg>
hipError_t launch_t(const GemmArgs& a, int splits, float* partial, bool reduce, hipStream_t s) {
  using TB = TA;
  constexpr int BM = Cfg::BM, BN = Cfg::BN;
  const int n_tiles = (a.N + BN - 1) / BN;
  int64_t m_tiles;
  if (a.g_off == nullptr) m_tiles = (a.M + BM - 1) / BM;
  else m_tiles = (a.max_rows + BM - 1) / BM + a.G;  // each group adds at most one partial tile
  int64_t total = m_tiles * n_tiles * (a.g_off ? 1 : splits);
  int64_t grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const uint64_t a_rows = a.g_off ? (uint64_t)a.a_nrows : (uint64_t)a.M;
  if (a_rows * a.lda * sizeof(TA) >= (1ull << 31) || (uint64_t)a.N * a.ldb * sizeof(TB) >= (1ull << 31))
    return hipErrorInvalidValue;
  if (a.b_scale) return hipErrorInvalidValue;  // fp8 weights: launch_gemm_fp8w
  float* part = splits > 1 ? partial : nullptr;
  if (part && BM * BN > 128 * 128) return hipErrorInvalidValue;  // partial tile must fit LDS
  // two weight matrices: dense, whole column tiles each, partials only
  if (a.B2 && (a.g_off || a.N0 <= 0 || a.N0 >= a.N || a.N0 % BN || !part || reduce ||
               (uint64_t)a.N0 * a.ldb * sizeof(TB) >= (1ull << 31)))
    return hipErrorInvalidValue;
  // residual: dense, whole 4-column groups, 16-byte aligned rows
  if (a.R && (a.g_off || a.N % 4 || a.ldr % 4 || a.ldr < a.N || a.act != kActNone ||
              (reinterpret_cast<uintptr_t>(a.R) & 15u) || (part && !reduce)))
    return hipErrorInvalidValue;
  // SwiGLU: whole column pairs, output N / 2 wide
  if (a.act == kActSwiGlu && (a.N % 4 || a.ldc < a.N / 2 || a.B2)) return hipErrorInvalidValue;
  if (a.act == kActSqRelu)
    gemm_tiled_kernel<Mma, TA, TOut, Cfg, kActSqRelu><<<dim3(grid), dim3(Cfg::NT), 0, s>>>(a, splits, part);
  else if (a.act == kActSwiGlu)
    gemm_tiled_kernel<Mma, TA, TOut, Cfg, kActSwiGlu><<<dim3(grid), dim3(Cfg::NT), 0, s>>>(a, splits, part);
  else
    gemm_tiled_kernel<Mma, TA, TOut, Cfg, kActNone><<<dim3(grid), dim3(Cfg::NT), 0, s>>>(a, splits, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !part || !reduce) return e;
  const int64_t n4 = (int64_t)a.M * (a.N / 4);
  const dim3 rg((n4 + 255) / 256);
  TOut* C = static_cast<TOut*>(a.C);
  if (a.act == kActSqRelu)
    splitk_reduce_kernel<TOut, kActSqRelu><<<rg, 256, 0, s>>>(part, splits, a.M, a.N, a.R, a.ldr, C, a.ldc);
  else if (a.act == kActSwiGlu)
    splitk_reduce_kernel<TOut, kActSwiGlu><<<rg, 256, 0, s>>>(part, splits, a.M, a.N, a.R, a.ldr, C, a.ldc);
  else
    splitk_reduce_kernel<TOut, kActNone><<<rg, 256, 0, s>>>(part, splits, a.M, a.N, a.R, a.ldr, C, a.ldc);
  return hipGetLastError();
}

// fp32 operands only with the small tiles; fp32 output (router logits,
// partials) with tiles of at most 128 x 256
template <typename Cfg>
hipError_t launch_tile(const GemmArgs& a, Dt a_dt, Dt out_dt, int splits, float* partial,
                       bool reduce, hipStream_t s) {
  // 32x32 MFMA blocks where the wave sub-tile holds at least 2 x 2 of them
  using MmaB = std::conditional_t<(Cfg::BM / Cfg::WGM >= 64 && Cfg::BN / Cfg::WGN >= 64),
                                  MmaBf16x32, MmaBf16>;
  if (a_dt == Dt::BF16) {
    if (out_dt == Dt::BF16) return launch_t<MmaB, uint16_t, uint16_t, Cfg>(a, splits, partial, reduce, s);
    if constexpr (Cfg::BM * Cfg::BN <= 128 * 256)
      return launch_t<MmaB, uint16_t, float, Cfg>(a, splits, partial, reduce, s);
    return hipErrorInvalidValue;
  }
  if constexpr (Cfg::BM * Cfg::BN <= 64 * 64)
    return launch_t<MmaF32, float, float, Cfg>(a, splits, partial, reduce, s);
  return hipErrorInvalidValue;
}

}  // namespace

int tiled_block_m(int tile) {
  switch (tile) {  // (fp32 layers run every tile index as Tile64)
    case 0: return Tile128::BM;
    case 1: return Tile64::BM;
    case 2: return Tile256::BM;
    default: return Tile128x256::BM;
  }
}

hipError_t launch_gemm_tiled(const GemmArgs& a, Dt a_dt, Dt out_dt, int tile, hipStream_t s,
                             int splits, float* partial, bool reduce) {
  if (a_dt == Dt::FP8) return hipErrorInvalidValue;  // fp8 weights: launch_gemm_fp8w, gemm_stream
  if (a_dt == Dt::F32 && out_dt != Dt::F32) return hipErrorInvalidValue;
  if (splits < 1 || (splits > 1 && (a.g_off != nullptr || partial == nullptr || a.N % 4)))
    return hipErrorInvalidValue;
  // fp32 layers (small) always take the 64 x 64 tile
  if (a_dt == Dt::F32) return launch_tile<Tile64>(a, a_dt, out_dt, splits, partial, reduce, s);
  switch (tile) {
    case 0: return launch_tile<Tile128>(a, a_dt, out_dt, splits, partial, reduce, s);
    case 1: return launch_tile<Tile64>(a, a_dt, out_dt, splits, partial, reduce, s);
    case 2: return launch_tile<Tile256>(a, a_dt, out_dt, splits, partial, reduce, s);
    case 3: return launch_tile<Tile128x256>(a, a_dt, out_dt, splits, partial, reduce, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lmoe
