// LDS-tiled MFMA GEMM, dense or grouped by expert, for gfx950.
//
// C[r][n] = act(scale[n] * sum_k A[arow(r)][k] * B[g][n][k])
//
// Used for the two projections (W_down: u = x W_down^T, W_up: out = v W_up^T),
// the router logits (fp32 output) and, when experts receive many tokens, the
// grouped latent expert GEMMs (FC1 gathers token rows through token_of).
//
// Block tile BM x BN x 128 bytes of K, 256 threads = 4 waves in a 2 x 2
// arrangement, each wave computing (BM/2) x (BN/2) with 16x16 MFMA blocks.
// Global -> register -> LDS staging, double-buffered LDS (one barrier per K
// stage).  LDS rows are 8 chunks of 16 bytes; chunk c of row r is stored at
// position c ^ (r & 7) so that the 16 lanes reading one fragment column hit
// distinct banks and the 8 lanes writing one row do too.
#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

template <typename Mma, typename TA, typename TOut, int BM, int BN, int ACT, bool SCALE>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmArgs p) {
  constexpr int EPC = 16 / sizeof(TA);   // elements per 16-byte chunk
  constexpr int BKE = 8 * EPC;           // elements of K per stage (128 bytes)
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;
  __shared__ u32x4 As[2][BM * 8];
  __shared__ u32x4 Bs[2][BN * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n_tiles = (p.N + BN - 1) / BN;

  // ---- which tile
  int g = 0, row0, rows, col0;
  if (p.g_off == nullptr) {
    const int total = ((p.M + BM - 1) / BM) * n_tiles;
    const int item = xcd_contiguous_item(blockIdx.x, gridDim.x, total);
    if (item < 0) return;
    row0 = (item / n_tiles) * BM;
    col0 = (item % n_tiles) * BN;
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

  const TA* A = static_cast<const TA*>(p.A);
  const TA* B = static_cast<const TA*>(p.B) + (int64_t)g * p.b_gstride;
  const int K = p.K;
  const int nk = (K + BKE - 1) / BKE;

  // ---- per-thread staging coordinates (fixed over K)
  const TA* a_src[ACH];
  int a_dst[ACH], a_k[ACH];
  bool a_ok[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int q = tid + i * 256, r = q >> 3, c = q & 7;
    a_ok[i] = r < rows;
    int64_t arow = 0;
    if (a_ok[i]) arow = p.a_rows ? p.a_rows[row0 + r] : row0 + r;
    a_src[i] = A + arow * p.lda + c * EPC;
    a_k[i] = c * EPC;
    a_dst[i] = r * 8 + (c ^ (r & 7));
  }
  const TA* b_src[BCH];
  int b_dst[BCH], b_k[BCH];
  bool b_ok[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int q = tid + i * 256, r = q >> 3, c = q & 7;
    b_ok[i] = col0 + r < p.N;
    b_src[i] = B + (int64_t)(b_ok[i] ? col0 + r : 0) * p.ldb + c * EPC;
    b_k[i] = c * EPC;
    b_dst[i] = r * 8 + (c ^ (r & 7));
  }

  u32x4 ra[ACH], rb[BCH];
  const void* zp = g_zero_chunk;
  auto load_stage = [&](int kt) {
    const int kb = kt * BKE;
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      ra[i] = load_chunk((a_ok[i] && kb + a_k[i] < K) ? static_cast<const void*>(a_src[i] + kb) : zp);
#pragma unroll
    for (int i = 0; i < BCH; ++i)
      rb[i] = load_chunk((b_ok[i] && kb + b_k[i] < K) ? static_cast<const void*>(b_src[i] + kb) : zp);
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) As[buf][a_dst[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) Bs[buf][b_dst[i]] = rb[i];
  };

  f32x4_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, fq = lane >> 4;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    load_stage(kt + 1);  // unconditional: past the end of K it reads the zero chunk
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = ks * 4 + fq;
      u32x4 af[MI], bfr[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm * WM + i * 16 + fr;
        af[i] = As[buf][r * 8 + (c ^ (r & 7))];
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int r = wn * WN + j * 16 + fr;
        bfr[j] = Bs[buf][r * 8 + (c ^ (r & 7))];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) Mma::mma(acc[i][j], af[i], bfr[j]);
    }
    store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  TOut* C = static_cast<TOut*>(p.C);
  const float* sc = SCALE ? p.b_scale + (int64_t)g * p.s_gstride : nullptr;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int col = col0 + wn * WN + j * 16 + fr;
    if (col >= p.N) continue;
    const float s = SCALE ? sc[col] : 1.f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wm * WM + i * 16 + fq * 4 + v;
        if (r < rows) {
          float val = acc[i][j][v];
          if (SCALE) val *= s;
          store_elem<TOut>(C + (int64_t)(row0 + r) * p.ldc + col, apply_act<ACT>(val));
        }
      }
    }
  }
}

template <typename Mma, typename TA, typename TOut, int BM, int BN>
hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
  const int n_tiles = (a.N + BN - 1) / BN;
  int64_t m_tiles;
  if (a.g_off == nullptr) m_tiles = (a.M + BM - 1) / BM;
  else m_tiles = (a.max_rows + BM - 1) / BM + a.G;  // each group adds at most one partial tile
  int64_t total = m_tiles * n_tiles;
  int64_t grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const bool scale = a.b_scale != nullptr;
  if (a.act == kActSqRelu) {
    if (scale) gemm_tiled_kernel<Mma, TA, TOut, BM, BN, kActSqRelu, true><<<dim3(grid), dim3(256), 0, s>>>(a);
    else gemm_tiled_kernel<Mma, TA, TOut, BM, BN, kActSqRelu, false><<<dim3(grid), dim3(256), 0, s>>>(a);
  } else {
    if (scale) gemm_tiled_kernel<Mma, TA, TOut, BM, BN, kActNone, true><<<dim3(grid), dim3(256), 0, s>>>(a);
    else gemm_tiled_kernel<Mma, TA, TOut, BM, BN, kActNone, false><<<dim3(grid), dim3(256), 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_tile(const GemmArgs& a, Dt a_dt, Dt out_dt, hipStream_t s) {
  if (a_dt == Dt::BF16) {
    if (out_dt == Dt::BF16) return launch_t<MmaBf16, uint16_t, uint16_t, BM, BN>(a, s);
    return launch_t<MmaBf16, uint16_t, float, BM, BN>(a, s);
  }
  return launch_t<MmaF32, float, float, BM, BN>(a, s);
}

}  // namespace

int tiled_block_m(int tile) { return tile == 0 ? 128 : 64; }

hipError_t launch_gemm_tiled(const GemmArgs& a, Dt a_dt, Dt out_dt, int tile, hipStream_t s) {
  if (a_dt == Dt::FP8) return hipErrorInvalidValue;  // fp8 weights go through the streaming kernel
  if (a_dt == Dt::F32 && out_dt != Dt::F32) return hipErrorInvalidValue;
  if (tile == 0) return launch_tile<128, 128>(a, a_dt, out_dt, s);
  return launch_tile<64, 64>(a, a_dt, out_dt, s);
}

}  // namespace lmoe
