// LDS-tiled MFMA GEMM, dense or grouped by expert, for gfx950.
//
// C[r][n] = act(scale[n] * sum_k A[arow(r)][k] * B[g][n][k])
//
// Used for the two projections (W_down: u = x W_down^T, W_up: out = v W_up^T),
// the router logits (fp32 output) and, when experts receive many tokens, the
// grouped latent expert GEMMs (FC1 gathers token rows through token_of).
//
// Block tile BM x BN, 256 threads = 4 waves in a 2 x 2 arrangement, each wave
// computing (BM/2) x (BN/2) with 16x16 MFMA blocks.  K advances in stages of
// 128 bytes per row.  Operands are read with raw buffer loads (32-bit
// offsets, out-of-range offsets read zero) into registers two stages ahead
// and written to one of two LDS buffers one stage ahead, so one barrier per
// stage separates the buffer being read from the one being filled.  LDS rows
// are 8 chunks of 16 bytes; chunk c of row r is stored at position c ^ (r & 7)
// so the 16 lanes reading one fragment column and the 8 lanes writing one
// row hit distinct banks.  The output tile leaves through LDS as 16-byte row
// chunks.
//
// Dense problems with too few tiles to fill the device split K: every split
// writes an fp32 partial tile and a reduction kernel adds the partials in a
// fixed order (deterministic), then scales, activates and converts.
#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

template <typename Mma, typename TA, typename TOut, int BM, int BN, int ACT, bool SCALE>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmArgs p, int splits, float* partial) {
  constexpr int EPC = 16 / sizeof(TA);   // elements per 16-byte chunk
  constexpr int BKE = 8 * EPC;           // elements of K per stage (128 bytes)
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;
  constexpr int STAGE = (BM + BN) * 8;   // chunks per LDS stage buffer
  __shared__ u32x4 smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
    g = lo;
    const int gs = p.g_off[g], ge = p.g_off[g + 1];
    row0 = gs + (mg - p.g_tiles[g]) * BM;
    rows = min(BM, ge - row0);
  }
  // K range of this split, in whole stages
  const int nk_all = (p.K + BKE - 1) / BKE;
  const int per = (nk_all + splits - 1) / splits;
  const int kt0 = kz * per;
  const int nk = max(0, min(nk_all, kt0 + per) - kt0);
  const int k_end = min(p.K, (kt0 + nk) * BKE);

  const TA* A = static_cast<const TA*>(p.A);
  const TA* B = static_cast<const TA*>(p.B) + (int64_t)g * p.b_gstride;
  const uint64_t a_rows_total = p.g_off ? (uint64_t)p.a_nrows : (uint64_t)p.M;
  const BufRsrc a_rsrc = make_rsrc(A, a_rows_total * p.lda * sizeof(TA));
  const BufRsrc b_rsrc = make_rsrc(B, (uint64_t)p.N * p.ldb * sizeof(TA));

  // ---- per-thread staging coordinates: chunk column sc_ of rows sr + 32 i
  const int sc_ = tid & 7;
  const int sr = tid >> 3;
  uint32_t a_off[ACH], b_off[BCH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int r = sr + 32 * i;
    int64_t arow = -1;
    if (r < rows) arow = p.a_rows ? p.a_rows[row0 + r] : row0 + r;
    a_off[i] = arow >= 0 ? static_cast<uint32_t>(arow * p.lda * sizeof(TA)) + sc_ * 16u : kOutOfRange;
  }
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int r = sr + 32 * i;
    b_off[i] = col0 + r < p.N ? static_cast<uint32_t>((int64_t)(col0 + r) * p.ldb * sizeof(TA)) +
                                    sc_ * 16u
                              : kOutOfRange;
  }

  u32x4 ra0[ACH], rb0[BCH], ra1[ACH], rb1[BCH];
#define LMOE_LOAD(kt, ra, rb)                                                           \
  do {                                                                                  \
    const int k_ = ((kt0 + (kt)) * BKE) + sc_ * EPC;                                    \
    const bool in_ = (kt) < nk && k_ < k_end;                                           \
    /* the stage offset is wave-uniform: keep it in an SGPR (buffer soffset) */         \
    const uint32_t so_ = __builtin_amdgcn_readfirstlane(                                \
        static_cast<uint32_t>((kt0 + (kt)) * BKE * sizeof(TA)));                        \
    _Pragma("unroll") for (int i = 0; i < ACH; ++i)                                     \
      ra[i] = buffer_load_chunk(a_rsrc, in_ ? a_off[i] : kOutOfRange, so_);             \
    _Pragma("unroll") for (int i = 0; i < BCH; ++i)                                     \
      rb[i] = buffer_load_chunk(b_rsrc, in_ ? b_off[i] : kOutOfRange, so_);             \
  } while (0)
#define LMOE_STORE(buf, ra, rb)                                                         \
  do {                                                                                  \
    u32x4* s_ = smem + (buf) * STAGE;                                                   \
    _Pragma("unroll") for (int i = 0; i < ACH; ++i) {                                   \
      const int r_ = sr + 32 * i;                                                       \
      s_[r_ * 8 + (sc_ ^ (r_ & 7))] = ra[i];                                            \
    }                                                                                   \
    _Pragma("unroll") for (int i = 0; i < BCH; ++i) {                                   \
      const int r_ = BM + sr + 32 * i;                                                  \
      s_[r_ * 8 + (sc_ ^ (r_ & 7))] = rb[i];                                            \
    }                                                                                   \
  } while (0)

  f32x4_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, fq = lane >> 4;
#define LMOE_COMPUTE(buf)                                                               \
  do {                                                                                  \
    const u32x4* s_ = smem + (buf) * STAGE;                                             \
    _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                  \
      const int c_ = ks * 4 + fq;                                                       \
      u32x4 af[MI], bfr[NI];                                                            \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                  \
        const int r_ = wm * WM + i * 16 + fr;                                           \
        af[i] = s_[r_ * 8 + (c_ ^ (r_ & 7))];                                           \
      }                                                                                 \
      _Pragma("unroll") for (int j = 0; j < NI; ++j) {                                  \
        const int r_ = BM + wn * WN + j * 16 + fr;                                      \
        bfr[j] = s_[r_ * 8 + (c_ ^ (r_ & 7))];                                          \
      }                                                                                 \
      _Pragma("unroll") for (int i = 0; i < MI; ++i)                                    \
      _Pragma("unroll") for (int j = 0; j < NI; ++j) Mma::mma(acc[i][j], af[i], bfr[j]); \
    }                                                                                   \
  } while (0)

  // stage kt: registers set kt%2 -> LDS buffer kt%2 one stage ahead; the loads
  // of stage kt+2 are issued before the multiplies of stage kt
  LMOE_LOAD(0, ra0, rb0);
  LMOE_LOAD(1, ra1, rb1);
  LMOE_STORE(0, ra0, rb0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    LMOE_LOAD(kt + 2, ra0, rb0);
    __builtin_amdgcn_sched_barrier(0);
    LMOE_COMPUTE(0);
    LMOE_STORE(1, ra1, rb1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    LMOE_LOAD(kt + 3, ra1, rb1);
    __builtin_amdgcn_sched_barrier(0);
    LMOE_COMPUTE(1);
    LMOE_STORE(0, ra0, rb0);
    __syncthreads();
  }
#undef LMOE_LOAD
#undef LMOE_STORE
#undef LMOE_COMPUTE

  // ---- epilogue through LDS: direct output (scale, act, convert) or fp32 partial
  const float* sc = SCALE ? p.b_scale + (int64_t)g * p.s_gstride : nullptr;
  if (partial == nullptr) {
    static_assert(BM * BN * sizeof(TOut) <= sizeof(smem), "output tile must fit LDS");
    TOut* Ct = reinterpret_cast<TOut*>(smem);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int colt = wn * WN + j * 16 + fr;
      const float s = (SCALE && col0 + colt < p.N) ? sc[col0 + colt] : 1.f;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float val = acc[i][j][v];
          if (SCALE) val *= s;
          store_elem<TOut>(Ct + (wm * WM + i * 16 + fq * 4 + v) * BN + colt, apply_act<ACT>(val));
        }
    }
    __syncthreads();
    constexpr int CPR = BN * sizeof(TOut) / 16;
    constexpr int EPO = 16 / sizeof(TOut);
    TOut* C = static_cast<TOut*>(p.C);
    // whole 16-byte chunks where the row stride keeps them aligned and the
    // chunk lies inside N; element stores otherwise (e.g. N = expert count)
    const bool aligned = (p.ldc % EPO) == 0;
    for (int q = tid; q < rows * CPR; q += 256) {
      const int r = q / CPR, ch = q % CPR;
      const int col = col0 + ch * EPO;
      TOut* dst = C + (int64_t)(row0 + r) * p.ldc + col;
      if (aligned && col + EPO <= p.N) {
        *reinterpret_cast<u32x4*>(dst) = reinterpret_cast<const u32x4*>(Ct)[q];
      } else {
        for (int e = 0; e < EPO && col + e < p.N; ++e) dst[e] = Ct[r * BN + ch * EPO + e];
      }
    }
  } else {
    static_assert(BM * BN * 4 <= sizeof(smem), "partial tile must fit LDS");
    float* Pt = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          Pt[(wm * WM + i * 16 + fq * 4 + v) * BN + wn * WN + j * 16 + fr] = acc[i][j][v];
    __syncthreads();
    constexpr int CPR = BN / 4;
    float* P = partial + (int64_t)kz * p.M * p.N;
    for (int q = tid; q < rows * CPR; q += 256) {
      const int r = q / CPR, ch = q % CPR;
      const int col = col0 + ch * 4;
      if (col < p.N)
        *reinterpret_cast<u32x4*>(P + (int64_t)(row0 + r) * p.N + col) =
            reinterpret_cast<const u32x4*>(Pt)[q];
    }
  }
}

// C[r][c] = act(scale[c] * sum_s P[s][r][c]), splits added in order.
template <typename TOut, int ACT, bool SCALE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int splits,
                                                            int M, int N, const float* __restrict__ scale,
                                                            TOut* __restrict__ C, int64_t ldc) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4 columns per thread
  const int64_t total = (int64_t)M * (N / 4);
  if (q >= total) return;
  const int r = static_cast<int>(q / (N / 4));
  const int c = static_cast<int>(q % (N / 4)) * 4;
  const int64_t mn = (int64_t)M * N;
  f32x4_t s = *reinterpret_cast<const f32x4_t*>(P + (int64_t)r * N + c);
  for (int z = 1; z < splits; ++z) s += *reinterpret_cast<const f32x4_t*>(P + z * mn + (int64_t)r * N + c);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float val = s[v];
    if (SCALE) val *= scale[c + v];
    store_elem<TOut>(C + (int64_t)r * ldc + c + v, apply_act<ACT>(val));
  }
}

template <typename Mma, typename TA, typename TOut, int BM, int BN>
hipError_t launch_t(const GemmArgs& a, int splits, float* partial, hipStream_t s) {
  const int n_tiles = (a.N + BN - 1) / BN;
  int64_t m_tiles;
  if (a.g_off == nullptr) m_tiles = (a.M + BM - 1) / BM;
  else m_tiles = (a.max_rows + BM - 1) / BM + a.G;  // each group adds at most one partial tile
  int64_t total = m_tiles * n_tiles * (a.g_off ? 1 : splits);
  int64_t grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const uint64_t a_rows = a.g_off ? (uint64_t)a.a_nrows : (uint64_t)a.M;
  if (a_rows * a.lda * sizeof(TA) >= (1ull << 31) || (uint64_t)a.N * a.ldb * sizeof(TA) >= (1ull << 31))
    return hipErrorInvalidValue;
  const bool scale = a.b_scale != nullptr;
  float* part = splits > 1 ? partial : nullptr;
  if (a.act == kActSqRelu) {
    if (scale) gemm_tiled_kernel<Mma, TA, TOut, BM, BN, kActSqRelu, true><<<dim3(grid), dim3(256), 0, s>>>(a, splits, part);
    else gemm_tiled_kernel<Mma, TA, TOut, BM, BN, kActSqRelu, false><<<dim3(grid), dim3(256), 0, s>>>(a, splits, part);
  } else {
    if (scale) gemm_tiled_kernel<Mma, TA, TOut, BM, BN, kActNone, true><<<dim3(grid), dim3(256), 0, s>>>(a, splits, part);
    else gemm_tiled_kernel<Mma, TA, TOut, BM, BN, kActNone, false><<<dim3(grid), dim3(256), 0, s>>>(a, splits, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !part) return e;
  const int64_t n4 = (int64_t)a.M * (a.N / 4);
  const dim3 rg((n4 + 255) / 256);
  TOut* C = static_cast<TOut*>(a.C);
  if (a.act == kActSqRelu) {
    if (scale) splitk_reduce_kernel<TOut, kActSqRelu, true><<<rg, 256, 0, s>>>(part, splits, a.M, a.N, a.b_scale, C, a.ldc);
    else splitk_reduce_kernel<TOut, kActSqRelu, false><<<rg, 256, 0, s>>>(part, splits, a.M, a.N, nullptr, C, a.ldc);
  } else {
    if (scale) splitk_reduce_kernel<TOut, kActNone, true><<<rg, 256, 0, s>>>(part, splits, a.M, a.N, a.b_scale, C, a.ldc);
    else splitk_reduce_kernel<TOut, kActNone, false><<<rg, 256, 0, s>>>(part, splits, a.M, a.N, nullptr, C, a.ldc);
  }
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_tile(const GemmArgs& a, Dt a_dt, Dt out_dt, int splits, float* partial,
                       hipStream_t s) {
  if (a_dt == Dt::BF16) {
    if (out_dt == Dt::BF16) return launch_t<MmaBf16, uint16_t, uint16_t, BM, BN>(a, splits, partial, s);
    return launch_t<MmaBf16, uint16_t, float, BM, BN>(a, splits, partial, s);
  }
  return launch_t<MmaF32, float, float, BM, BN>(a, splits, partial, s);
}

}  // namespace

int tiled_block_m(int tile) { return tile == 0 ? 128 : 64; }

hipError_t launch_gemm_tiled(const GemmArgs& a, Dt a_dt, Dt out_dt, int tile, hipStream_t s,
                             int splits, float* partial) {
  if (a_dt == Dt::FP8) return hipErrorInvalidValue;  // fp8 weights go through the streaming kernel
  if (a_dt == Dt::F32 && out_dt != Dt::F32) return hipErrorInvalidValue;
  if (splits < 1 || (splits > 1 && (a.g_off != nullptr || partial == nullptr || a.N % 4)))
    return hipErrorInvalidValue;
  if (tile == 0) return launch_tile<128, 128>(a, a_dt, out_dt, splits, partial, s);
  return launch_tile<64, 64>(a, a_dt, out_dt, splits, partial, s);
}

}  // namespace lmoe
