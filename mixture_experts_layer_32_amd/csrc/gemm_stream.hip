// Weight-streaming grouped GEMM for the latent experts when each expert
// receives few token copies (decode regime), for gfx950.
//
// C[r][n] = act(scale[g][n] * sum_k A[arow(r)][k] * W[g][n][k]),  r in group g
//
// With a few dozen rows per expert the GEMM is bound by reading the expert
// weights from HBM once, so the kernel is built around that stream:
//  - One workgroup per (expert, tile of 64 * NWB output columns); the tiles of
//    one expert are contiguous work items, hence on one XCD, sharing the
//    expert's token rows in that XCD's L2.
//  - Each wave streams its own 16 * NWB weight rows straight from global
//    memory into registers in the MFMA B-operand layout (4 lanes per weight
//    row, 16 contiguous bytes each, so a load instruction reads 64 contiguous
//    bytes of each of 16 rows and two consecutive ones complete 128-byte
//    lines); the next K stage of weights is in flight while the current one
//    is multiplied.
//  - The (at most 16 * MB_MAX) token rows of the expert are staged through LDS
//    per K stage (double-buffered), gathered through token_of for FC1: this is
//    the dispatch of the token copies, done without materialising them.
//  - fp8 (OCP E4M3) weights are widened to bf16 in registers (exact) and the
//    per-row scale is applied to the fp32 accumulator in the epilogue.
// Experts with more rows than one pass holds are processed in several passes
// (the weights are then streamed once per pass).
//
// Reduction-index assignment within a 256-byte stage of A (bf16, fp8
// weights): MFMA step s (32 indices) takes, for lane group q, the 8 indices
// starting at 64 * (s / 2) + 16 * q + 8 * (s % 2), so a lane owns 16
// consecutive indices of every 64 (one fp8 chunk, or two bf16 chunks).
#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

template <typename TA> struct StreamTraits;
template <> struct StreamTraits<uint16_t> {  // bf16 activations
  static constexpr int EPC = 8;              // elements per 16-byte chunk
  static constexpr int KSTEP = 32;           // reduction indices per MFMA
  __device__ __forceinline__ static int elem_of(int s, int q) {
    return 64 * (s >> 1) + 16 * q + 8 * (s & 1);
  }
};
template <> struct StreamTraits<float> {     // fp32 activations and weights
  static constexpr int EPC = 4;
  static constexpr int KSTEP = 16;
  __device__ __forceinline__ static int elem_of(int s, int q) { return 16 * s + 4 * q; }
};

constexpr int kStageChunks = 16;  // 16-byte chunks of A per row per K stage (256 bytes)

// MB_MAX m-blocks of 16 rows per pass, NWB n-blocks of 16 weight rows per wave.
template <typename Mma, typename TA, typename TW, typename TOut, int MB_MAX, int NWB, int ACT,
          bool SCALE>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs p) {
  using Tr = StreamTraits<TA>;
  constexpr int EPC = Tr::EPC;
  constexpr int KE = kStageChunks * EPC;    // reduction elements per stage
  constexpr int NS = KE / Tr::KSTEP;        // MFMA steps per stage (4)
  constexpr bool FP8 = sizeof(TW) == 1;
  constexpr int NLD = FP8 ? NS / 2 : NS;    // 16-byte weight loads per n-block per stage
  constexpr int MROWS = MB_MAX * 16;
  constexpr int NT = 4 * NWB * 16;          // output columns per workgroup
  static_assert(NS % 2 == 0, "stage must hold whole fp8 chunks");

  __shared__ u32x4 As[2][MROWS * kStageChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;

  const int n_tiles = (p.N + NT - 1) / NT;
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x, p.G * n_tiles);
  if (item < 0) return;
  const int g = item / n_tiles;
  const int col0 = (item % n_tiles) * NT;
  const int gs = p.g_off[g];
  const int cnt = p.g_off[g + 1] - gs;
  if (cnt <= 0) return;

  const int K = p.K;
  const int nst = (K + KE - 1) / KE;
  const TA* __restrict__ A = static_cast<const TA*>(p.A);

  // weight rows of this lane (one per n-block), clamped into the matrix
  const TW* wrow[NWB];
#pragma unroll
  for (int nb = 0; nb < NWB; ++nb) {
    int n = col0 + wave * NWB * 16 + nb * 16 + fr;
    n = n < p.N ? n : p.N - 1;
    wrow[nb] = static_cast<const TW*>(p.B) + (int64_t)g * p.b_gstride + (int64_t)n * p.ldb;
  }
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  TOut* C = static_cast<TOut*>(p.C);
  const float* sc = SCALE ? p.b_scale + (int64_t)g * p.s_gstride : nullptr;

  // A staging: thread owns chunk column ac of rows ar0 + 16 i
  const int ac = tid & 15;
  const int ar0 = tid >> 4;

  for (int p0 = 0; p0 < cnt; p0 += MROWS) {
    const int rows = min(MROWS, cnt - p0);
    const int nmb = (rows + 15) >> 4;

    int arow[MB_MAX];  // source row of A for each staged row, -1 = padding
#pragma unroll
    for (int i = 0; i < MB_MAX; ++i) {
      const int r = ar0 + 16 * i;
      arow[i] = r < rows ? (p.a_rows ? p.a_rows[gs + p0 + r] : gs + p0 + r) : -1;
    }

    f32x4_t acc[MB_MAX][NWB];
#pragma unroll
    for (int i = 0; i < MB_MAX; ++i)
#pragma unroll
      for (int j = 0; j < NWB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[MB_MAX];
    u32x4 b0[NWB][NLD], b1[NWB][NLD];

#define LMOE_LOAD_A(st)                                                                      \
  do {                                                                                       \
    const int k_ = (st) * KE + ac * EPC;                                                     \
    _Pragma("unroll") for (int i = 0; i < MB_MAX; ++i) {                                     \
      const bool ok_ = arow[i] >= 0 && k_ < K;                                               \
      const u32x4 v_ = *reinterpret_cast<const u32x4*>(                                      \
          A + (ok_ ? (int64_t)arow[i] * p.lda + k_ : (int64_t)0));                            \
      ra[i] = ok_ ? v_ : zero;                                                               \
    }                                                                                        \
  } while (0)
#define LMOE_STORE_A(buf)                                                                    \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < MB_MAX; ++i) {                                     \
      const int r_ = ar0 + 16 * i;                                                           \
      As[buf][r_ * kStageChunks + (ac ^ (r_ & 15))] = ra[i];                                 \
    }                                                                                        \
  } while (0)
#define LMOE_LOAD_W(st, br)                                                                  \
  do {                                                                                       \
    _Pragma("unroll") for (int nb = 0; nb < NWB; ++nb)                                       \
    _Pragma("unroll") for (int j = 0; j < NLD; ++j) {                                        \
      const int k_ = (st) * KE + (FP8 ? 64 * j + 16 * fq : Tr::elem_of(j, fq));             \
      const u32x4 v_ = *reinterpret_cast<const u32x4*>(wrow[nb] + (k_ < K ? k_ : 0));        \
      br[nb][j] = k_ < K ? v_ : zero;                                                        \
    }                                                                                        \
  } while (0)
#define LMOE_COMPUTE(buf, br)                                                                \
  do {                                                                                       \
    _Pragma("unroll") for (int s = 0; s < NS; ++s) {                                         \
      u32x4 bfr[NWB];                                                                        \
      _Pragma("unroll") for (int nb = 0; nb < NWB; ++nb) {                                   \
        if constexpr (FP8) {                                                                 \
          u32x4 lo_, hi_;                                                                    \
          fp8_chunk_to_bf16(br[nb][s >> 1], lo_, hi_);                                       \
          bfr[nb] = (s & 1) ? hi_ : lo_;                                                     \
        } else {                                                                             \
          bfr[nb] = br[nb][s];                                                               \
        }                                                                                    \
      }                                                                                      \
      const int c_ = Tr::elem_of(s, fq) / EPC;                                               \
      _Pragma("unroll") for (int mb = 0; mb < MB_MAX; ++mb) {                                \
        if (mb < nmb) {                                                                      \
          const int r_ = mb * 16 + fr;                                                       \
          const u32x4 af_ = As[buf][r_ * kStageChunks + (c_ ^ (r_ & 15))];                   \
          _Pragma("unroll") for (int nb = 0; nb < NWB; ++nb) Mma::mma(acc[mb][nb], af_, bfr[nb]); \
        }                                                                                    \
      }                                                                                      \
    }                                                                                        \
  } while (0)

    // prologue: A then W of stage 0 (A is waited on first, W stays in flight)
    LMOE_LOAD_A(0);
    LMOE_LOAD_W(0, b0);
    LMOE_STORE_A(0);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
      // even stage: compute from b0 / LDS buffer 0, prefetch stage st+1 into b1
      if (st + 1 < nst) { LMOE_LOAD_A(st + 1); LMOE_LOAD_W(st + 1, b1); }
      LMOE_COMPUTE(0, b0);
      if (st + 1 < nst) LMOE_STORE_A(1);
      __syncthreads();
      if (st + 1 >= nst) break;
      // odd stage: compute from b1 / LDS buffer 1, prefetch stage st+2 into b0
      if (st + 2 < nst) { LMOE_LOAD_A(st + 2); LMOE_LOAD_W(st + 2, b0); }
      LMOE_COMPUTE(1, b1);
      if (st + 2 < nst) LMOE_STORE_A(0);
      __syncthreads();
    }
#undef LMOE_LOAD_A
#undef LMOE_STORE_A
#undef LMOE_LOAD_W
#undef LMOE_COMPUTE

    // epilogue: accumulator lane layout C[4*fq + v][fr] of each 16x16 block
#pragma unroll
    for (int nb = 0; nb < NWB; ++nb) {
      const int col = col0 + wave * NWB * 16 + nb * 16 + fr;
      if (col >= p.N) continue;
      const float s = SCALE ? sc[col] : 1.f;
#pragma unroll
      for (int mb = 0; mb < MB_MAX; ++mb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = mb * 16 + fq * 4 + v;
          if (r < rows) {
            float val = acc[mb][nb][v];
            if (SCALE) val *= s;
            store_elem<TOut>(C + (int64_t)(gs + p0 + r) * p.ldc + col, apply_act<ACT>(val));
          }
        }
      }
    }
  }
}

template <typename Mma, typename TA, typename TW, typename TOut, int MB>
hipError_t launch_s(const GemmArgs& a, hipStream_t s) {
  constexpr int NWB = 2;
  constexpr int NT = 4 * NWB * 16;
  const int64_t n_tiles = (a.N + NT - 1) / NT;
  const int64_t total = n_tiles * a.G;
  const int64_t grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const bool scale = a.b_scale != nullptr;
  if (a.act == kActSqRelu) {
    if (scale) gemm_stream_kernel<Mma, TA, TW, TOut, MB, NWB, kActSqRelu, true><<<dim3(grid), dim3(256), 0, s>>>(a);
    else gemm_stream_kernel<Mma, TA, TW, TOut, MB, NWB, kActSqRelu, false><<<dim3(grid), dim3(256), 0, s>>>(a);
  } else {
    if (scale) gemm_stream_kernel<Mma, TA, TW, TOut, MB, NWB, kActNone, true><<<dim3(grid), dim3(256), 0, s>>>(a);
    else gemm_stream_kernel<Mma, TA, TW, TOut, MB, NWB, kActNone, false><<<dim3(grid), dim3(256), 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int MB>
hipError_t launch_mb(const GemmArgs& a, Dt a_dt, Dt w_dt, Dt out_dt, hipStream_t s) {
  if (a_dt == Dt::F32) {
    if (w_dt != Dt::F32 || out_dt != Dt::F32) return hipErrorInvalidValue;
    return launch_s<MmaF32, float, float, float, MB>(a, s);
  }
  if (out_dt != Dt::BF16) return hipErrorInvalidValue;
  if (w_dt == Dt::BF16) return launch_s<MmaBf16, uint16_t, uint16_t, uint16_t, MB>(a, s);
  if (w_dt == Dt::FP8) return launch_s<MmaBf16, uint16_t, uint8_t, uint16_t, MB>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_stream(const GemmArgs& a, Dt a_dt, Dt w_dt, Dt out_dt, int mb_max,
                              hipStream_t s) {
  if (mb_max <= 4) return launch_mb<4>(a, a_dt, w_dt, out_dt, s);
  return launch_mb<8>(a, a_dt, w_dt, out_dt, s);
}

}  // namespace lmoe
