// Grouped expert GEMM over fp8 expert weights, gfx950: OCP E4M3 weight
// bytes with one fp32 scale per weight row, bf16 token rows and output,
// fp32 accumulation.  For experts with a few dozen to about a hundred rows
// (large-batch decode of fine-grained MoEs), where reading the weights from
// HBM is the bound.
//
// C[r][n] = act(s_g[n] * sum_k A[arow(r)][k] * B_g[n][k]) for the rows r of
// each expert g (rows g_off[g] .. g_off[g+1]); FC1 gathers its A rows
// through a_rows, FC2 reads them in place.
//
// A workgroup of 4 waves computes a tile of 96 rows x 256 columns: wave w
// owns columns 64 w .. 64 w + 63 (four 16-column n-blocks) over all 96 rows
// (six 16-row m-blocks), in 16x16x32 bf16 MFMA blocks.  Each weight byte is
// used by one wave only, so the weights go from global memory straight into
// that wave's registers, three K stages (of 64) ahead of the one being
// multiplied: the weight bytes in flight per compute unit (two workgroups,
// 8 waves x 3 stages x 4 KB) are not bounded by LDS.  The token rows, which
// all 4 waves read, pass through a double-buffered LDS stage: loaded into
// registers two stages ahead and written to LDS after the current stage's
// MFMAs.  Every load is an ordinary buffer load the compiler sees, so its
// waits are exact: issued in the order (A stage k+2, B stage k+3) per
// stage, the wait for stage k's weights leaves three stages of weights in
// flight.
//
// Weights are widened to bf16 right before the MFMA with the gfx950 scaled
// conversion at scale 1 (exact: every E4M3 value is a bf16 value); the row
// scale joins in the epilogue, before the activation and the one rounding
// to bf16, as in the LDS-tiled kernel.  K-element assignment: in a 64-K
// stage, lane (n, q) (n = lane % 16, q = lane / 16) loads weight bytes
// [16 q, 16 q + 16) of row n of each n-block, so one load instruction reads
// 16 rows x 64 contiguous bytes (half the L2 requests of a 32-row MFMA
// layout, whose rows would get 32 bytes each); k-step s (of 32) uses bytes
// 8 s .. 8 s + 7, and the token fragments of k-step s read the same K
// elements (8-element chunk 2 q + s).  Only the pairing of the two
// operands matters for the sum.
//
// The epilogue stages one 16-row block row of a wave's columns in LDS and
// stores 16-byte chunks through a buffer resource whose range ends at the
// tile's last row (rows past it are dropped by the range check).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

constexpr int kF8NT = 256;                  // 4 waves
constexpr int kF8BM = 96;                   // rows per tile (6 m-blocks of 16)
constexpr int kF8BN = 256;                  // columns per tile (64 per wave)
constexpr int kF8KS = 64;                   // K elements per stage
constexpr int kF8AC = kF8KS / 8;            // 16-byte A chunks per row per stage (8)
constexpr int kF8ANum = kF8BM * kF8AC / kF8NT;  // A chunks per thread per stage (3)
constexpr int kF8DB = 4;                    // weight register stages (3 ahead)
constexpr int kF8OutLd = 64 + 8;            // staged output row (bf16 elements)
constexpr int kF8MB = kF8BM / 16;           // m-blocks (6)
constexpr int kF8NB = 4;                    // n-blocks of a wave
static_assert(kF8BM * kF8AC % kF8NT == 0, "A stage splits over the threads");

__device__ __forceinline__ int f8_swz(int r) { return (r >> 1) & 7; }

// 8 E4M3 bytes (2 dwords) -> 8 bf16 (one MFMA operand), exact
__device__ __forceinline__ u32x4 f8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true))};
}

// BANDS: the weights come as the packed 16-row bands, read non-temporally
// (each load instruction reads 1 KB in one piece and each byte once:
// 3 % faster per GEMM); row-major weights keep the default policy (a
// 128-byte line of a row is read by the instructions of two stages)
template <int ACT, bool SCALE, bool BANDS>
__global__ __launch_bounds__(kF8NT, 2) void gemm_fp8w_kernel(GemmArgs p) {
  __shared__ u32x4 sa[2][kF8BM * kF8AC];    // token stages, 2 x 12 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, nrow = lane & 15;

  // ---- the tile: (expert, 96-row tile, 256-column tile)
  const int n_tiles = (p.N + kF8BN - 1) / kF8BN;
  const int total = __builtin_amdgcn_readfirstlane(p.g_tiles[p.G]) * n_tiles;
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x, total);
  if (item < 0) return;
  const int mg = item / n_tiles;
  const int col0 = (item % n_tiles) * kF8BN;
  int lo = 0, hi = p.G - 1;  // last expert whose first row tile is <= mg
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.g_tiles[mid] <= mg) lo = mid; else hi = mid - 1;
  }
  const int g = __builtin_amdgcn_readfirstlane(lo);
  const int row0 = __builtin_amdgcn_readfirstlane(p.g_off[g]) +
                   (mg - __builtin_amdgcn_readfirstlane(p.g_tiles[g])) * kF8BM;
  const int rows = min(kF8BM, __builtin_amdgcn_readfirstlane(p.g_off[g + 1]) - row0);
  const int K = p.K;
  const int nk = (K + kF8KS - 1) / kF8KS;

  const BufRsrc a_rsrc = make_rsrc(p.A, (uint64_t)p.a_nrows * p.lda * 2);
  const uint8_t* B = static_cast<const uint8_t*>(p.B) + (int64_t)g * p.b_gstride;
  const BufRsrc b_rsrc = make_rsrc(B, (uint64_t)p.N * p.ldb);

  // A chunks of this thread: chunk q = j 256 + tid of the stage, row q / 8,
  // 8-element chunk q % 8, at LDS position row 8 + (chunk ^ swz(row))
  uint32_t a_off[kF8ANum];
  int a_k[kF8ANum], a_pos[kF8ANum];
#pragma unroll
  for (int j = 0; j < kF8ANum; ++j) {
    const int q = j * kF8NT + tid;
    const int r = q / kF8AC, c = q % kF8AC;
    a_k[j] = 8 * c;
    a_pos[j] = r * kF8AC + (c ^ f8_swz(r));
    int64_t arow = -1;
    if (r < rows) arow = p.a_rows ? p.a_rows[row0 + r] : row0 + r;
    a_off[j] = arow >= 0 ? static_cast<uint32_t>(arow * p.lda * 2) + 16u * c : kOutOfRange;
  }
  // weight rows of this lane: n-block j, row nrow; bytes 16 q4 .. of a stage
  // (banded B: the n-block's 16 rows x 64 bytes of a stage are one block)
  uint32_t b_off[kF8NB];
#pragma unroll
  for (int j = 0; j < kF8NB; ++j) {
    const int n = col0 + 64 * wave + 16 * j + nrow;
    const uint32_t o = p.b_bands ? static_cast<uint32_t>((n - nrow) * p.ldb) + 64u * nrow + 16u * q4
                                 : static_cast<uint32_t>(n * p.ldb) + 16u * q4;
    b_off[j] = n < p.N ? o : kOutOfRange;
  }
  const int b_step = p.b_bands ? 16 * kF8KS : kF8KS;   // bytes between K stages

  u32x4 areg[2][kF8ANum];       // token chunks, two stages
  u32x4 breg[kF8DB][kF8NB];     // weights [stage slot][n-block]
  auto load_a = [&](int kt, u32x4 (&dst)[kF8ANum]) {
    const int kb = kt * kF8KS;
#pragma unroll
    for (int j = 0; j < kF8ANum; ++j) {
      const bool in = a_off[j] != kOutOfRange && kb + a_k[j] < K;
      dst[j] = buffer_load_chunk(a_rsrc, in ? a_off[j] + 2u * kb : kOutOfRange, 0u);
    }
  };
  auto load_b = [&](int kt, u32x4 (&dst)[kF8NB]) {
    const int kb = kt * kF8KS;
#pragma unroll
    for (int j = 0; j < kF8NB; ++j) {
      const bool in = b_off[j] != kOutOfRange && kb + 16 * q4 < K;
      dst[j] = buffer_load_chunk<BANDS ? kCpolNonTemporal : kCpolDefault>(
          b_rsrc, in ? b_off[j] + kt * b_step : kOutOfRange, 0u);
    }
  };
  auto store_a = [&](const u32x4 (&src)[kF8ANum], int buf) {
#pragma unroll
    for (int j = 0; j < kF8ANum; ++j) sa[buf][a_pos[j]] = src[j];
  };

  f32x4_t acc[kF8MB][kF8NB];
#pragma unroll
  for (int i = 0; i < kF8MB; ++i)
#pragma unroll
    for (int j = 0; j < kF8NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one stage: 2 k-steps of 24 MFMAs; token fragments from LDS buffer buf,
  // weights from the register slot
  auto compute = [&](int buf, const u32x4 (&w)[kF8NB]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 2 * q4 + s;
      u32x4 fb[kF8NB];
#pragma unroll
      for (int j = 0; j < kF8NB; ++j)
        fb[j] = s ? f8x8_to_bf16x8(w[j].z, w[j].w) : f8x8_to_bf16x8(w[j].x, w[j].y);
#pragma unroll
      for (int i = 0; i < kF8MB; ++i) {
        const int r = 16 * i + nrow;
        const u32x4 fa = sa[buf][r * kF8AC + (c ^ f8_swz(r))];
#pragma unroll
        for (int j = 0; j < kF8NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, fb[j]), __builtin_bit_cast(bf16x8_t, fa), acc[i][j],
              0, 0, 0);
      }
    }
  };

  // ---- prologue: tokens of stages 0 and 1, weights of stages 0 .. 2;
  // stage 0's tokens into LDS buffer 0
  load_a(0, areg[0]);
  load_b(0, breg[0]);
  load_a(1, areg[1]);
  load_b(1, breg[1]);
  load_b(2, breg[2]);
  store_a(areg[0], 0);
  __syncthreads();

  // ---- main loop, 4 stages per pass (static register slots): stage kt
  // issues tokens kt + 2 and weights kt + 3, multiplies stage kt, then writes
  // stage kt + 1's tokens to the other LDS buffer
#define F8_STAGE(t)                                                             \
  do {                                                                          \
    const int kt = kt0 + (t);                                                   \
    load_a(kt + 2, areg[(t) & 1]);                                              \
    load_b(kt + 3, breg[((t) + 3) & 3]);                                        \
    if (kt < nk) compute((t) & 1, breg[(t) & 3]);                               \
    store_a(areg[((t) + 1) & 1], ((t) + 1) & 1);                                \
    __syncthreads();                                                            \
  } while (0)
  for (int kt0 = 0; kt0 < nk; kt0 += 4) {
    F8_STAGE(0);
    F8_STAGE(1);
    F8_STAGE(2);
    F8_STAGE(3);
  }
#undef F8_STAGE

  // ---- epilogue: per m-block, the wave's 16 x 64 outputs (16 x 32 with
  // SwiGLU) scaled, activated and rounded to bf16 into its staging area
  // (the token buffers, free now), then stored as 16-byte chunks.  Lane
  // (m, q) holds row m of the block and columns 4 q .. 4 q + 3 of each
  // n-block (the blocks are computed transposed).
  constexpr bool GLU = ACT == kActSwiGlu;
  constexpr int OW = GLU ? 32 : 64;          // output columns of a wave
  constexpr int CPR = OW / 8;                // 16-byte chunks per staged row
  constexpr int RPS = 64 / CPR;              // rows per wave store
  uint16_t* stg = reinterpret_cast<uint16_t*>(&sa[0][0]) + wave * 16 * kF8OutLd;
  const int n_out = GLU ? p.N / 2 : p.N;
  const int ocol0 = (GLU ? col0 / 2 : col0) + wave * OW;
  const uint32_t ldc2 = static_cast<uint32_t>(p.ldc) * 2;
  const BufRsrc c_rsrc = make_rsrc(p.C, static_cast<uint64_t>(row0 + rows) * ldc2);
  const int srow = lane / CPR, sch = lane % CPR;
  const bool col_in = ocol0 + 8 * sch < n_out;   // N % 16 == 0: whole chunks
  const uint32_t c_off = static_cast<uint32_t>(row0 + srow) * ldc2 +
                         static_cast<uint32_t>(ocol0 + 8 * sch) * 2;
  // the scales of this lane's 4 columns of each n-block
  f32x4_t sc4[kF8NB];
  if constexpr (SCALE) {
    const BufRsrc s_rsrc =
        make_rsrc(p.b_scale + (int64_t)g * p.s_gstride, static_cast<uint64_t>(p.N) * 4);
#pragma unroll
    for (int j = 0; j < kF8NB; ++j) {
      const int n = col0 + 64 * wave + 16 * j + 4 * q4;
      sc4[j] = __builtin_bit_cast(
          f32x4_t, buffer_load_chunk(s_rsrc, n < p.N ? 4u * n : kOutOfRange, 0u));
    }
  }
  __syncthreads();   // every wave is done with the token buffers
#pragma unroll
  for (int i = 0; i < kF8MB; ++i) {
#pragma unroll
    for (int j = 0; j < kF8NB; ++j) {
      const int c = 16 * j + 4 * q4;   // column within the wave's 64
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = acc[i][j][e];
        if constexpr (SCALE) v[e] *= sc4[j][e];
        if constexpr (!GLU) v[e] = apply_act<ACT>(v[e]);
      }
      if constexpr (GLU) {
        *reinterpret_cast<uint32_t*>(stg + nrow * kF8OutLd + c / 2) =
            pack_bf16x2(swiglu(v[0], v[1]), swiglu(v[2], v[3]));
      } else {
        *reinterpret_cast<uint2*>(stg + nrow * kF8OutLd + c) =
            uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
#pragma unroll
    for (int u = 0; u < 16 / RPS; ++u) {
      const u32x4 val =
          *reinterpret_cast<const u32x4*>(stg + (u * RPS + srow) * kF8OutLd + sch * 8);
      const uint32_t off = c_off + static_cast<uint32_t>(16 * i + u * RPS) * ldc2;
      // non-temporal: the output is read again only by the next kernel
      // (FC1 8 %, FC2 4 % faster)
      __builtin_amdgcn_raw_buffer_store_b128(val, c_rsrc, col_in ? off : kOutOfRange, 0,
                                             kCpolNonTemporal);
    }
  }
}

}  // namespace

bool gemm_fp8w_fits(int N, int K, int G) {
  return N > 0 && K > 0 && N % 16 == 0 && K % 16 == 0 && G >= 1 && G <= 8 * kF8NT;
}

int fp8w_block_m() { return kF8BM; }

hipError_t launch_gemm_fp8w(const GemmArgs& a, hipStream_t s) {
  if (a.g_off == nullptr || a.g_tiles == nullptr || !gemm_fp8w_fits(a.N, a.K, a.G) || a.B2 || a.R ||
      a.b_mx || a.a_nrows <= 0 || a.max_rows <= 0 || a.G < 1)
    return hipErrorInvalidValue;
  if (a.b_bands && (a.ldb != a.K || a.K % kF8KS)) return hipErrorInvalidValue;
  if (a.act == kActSwiGlu && (a.N % 32 || a.ldc < a.N / 2)) return hipErrorInvalidValue;
  if (a.act != kActSwiGlu && a.ldc < a.N) return hipErrorInvalidValue;
  // 32-bit buffer offsets: A, one expert's weights, C (max_rows bounds its rows)
  if ((uint64_t)a.a_nrows * a.lda * 2 >= (1ull << 31) || (uint64_t)a.N * a.ldb >= (1ull << 31) ||
      (uint64_t)a.max_rows * a.ldc * 2 >= (1ull << 31))
    return hipErrorInvalidValue;
  const int n_tiles = (a.N + kF8BN - 1) / kF8BN;
  const int64_t m_tiles = (a.max_rows + kF8BM - 1) / kF8BM + a.G;  // each expert adds at most one partial tile
  const int64_t grid = (m_tiles * n_tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const bool sc = a.b_scale != nullptr, bands = a.b_bands != 0;
  const dim3 g3(static_cast<unsigned>(grid)), b3(kF8NT);
  auto go = [&](auto act) {
    constexpr int ACT = decltype(act)::value;
    if (sc && bands) gemm_fp8w_kernel<ACT, true, true><<<g3, b3, 0, s>>>(a);
    else if (sc) gemm_fp8w_kernel<ACT, true, false><<<g3, b3, 0, s>>>(a);
    else if (bands) gemm_fp8w_kernel<ACT, false, true><<<g3, b3, 0, s>>>(a);
    else gemm_fp8w_kernel<ACT, false, false><<<g3, b3, 0, s>>>(a);
  };
  if (a.act == kActSqRelu) go(std::integral_constant<int, kActSqRelu>{});
  else if (a.act == kActSwiGlu) go(std::integral_constant<int, kActSwiGlu>{});
  else go(std::integral_constant<int, kActNone>{});
  return hipGetLastError();
}

}  // namespace lmoe
