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
//    memory into registers in the MFMA B-operand layout with raw buffer
//    loads: 4 lanes per weight row side by side, so one load instruction
//    reads 64 contiguous bytes of each of 16 rows.  The next K stage of
//    weights is in flight while the current one is multiplied.
//  - The (at most 16 * MB_MAX) token rows of the expert are staged through LDS
//    per K stage (double-buffered), gathered through token_of for FC1: this is
//    the dispatch of the token copies, done without materialising them.
//  - fp8 (OCP E4M3) weights are widened to bf16 in registers (exact) and the
//    per-row scale is applied to the fp32 accumulator in the epilogue.
// Experts with more rows than one pass holds are processed in several passes
// (the weights are then streamed once per pass).
//
// Out-of-range buffer offsets read as zero without a memory request: padding
// token rows, token chunks past the end of K and the weight prefetch past the
// last stage use that, so no select on loaded data delays a wait.  Weight
// chunks past the end of K inside the last stage (K not a multiple of the
// stage) read the next weight row or zero; they meet zero token values.
// Every weight offset is carried in the per-lane offset, which is what the
// range check applies to.
#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

// Reduction indices, within a K stage, that lane group q supplies to MFMA
// step s.  Every weight load instruction then reads 64 contiguous bytes of
// each of its 16 weight rows (the 4 groups side by side).
template <typename TA, typename TW> struct StreamTraits;
template <> struct StreamTraits<uint16_t, uint16_t> {  // bf16 tokens, bf16 weights
  static constexpr int EPC = 8;                         // elements per 16-byte chunk
  static constexpr int KSTEP = 32;                      // reduction indices per MFMA
  __device__ __forceinline__ static int elem_of(int s, int q) { return 32 * s + 8 * q; }
};
template <> struct StreamTraits<uint16_t, uint8_t> {   // bf16 tokens, fp8 weights:
  static constexpr int EPC = 8;                         // a lane owns the 16 consecutive
  static constexpr int KSTEP = 32;                      // indices of one fp8 chunk, used
  __device__ __forceinline__ static int elem_of(int s, int q) {  // by steps 2j and 2j+1
    return 64 * (s >> 1) + 16 * q + 8 * (s & 1);
  }
};
template <> struct StreamTraits<float, float> {        // fp32 tokens and weights
  static constexpr int EPC = 4;
  static constexpr int KSTEP = 16;
  __device__ __forceinline__ static int elem_of(int s, int q) { return 16 * s + 4 * q; }
};

#ifndef LMOE_W_CPOL
#define LMOE_W_CPOL kCpolDefault
#endif

constexpr int kStageChunks = 16;  // 16-byte chunks of A per row per K stage (256 bytes)

// K stages of weights requested ahead.  An fp8 stage is half the bytes of a
// bf16 one and its registers a quarter (one n-block), so fp8 looks further
// ahead to keep as many weight bytes in flight.
#ifndef LMOE_W_DEPTH
#define LMOE_W_DEPTH 1
#endif
#ifndef LMOE_W_DEPTH_FP8
#define LMOE_W_DEPTH_FP8 4
#endif
template <typename TW>
constexpr int stream_w_depth() { return sizeof(TW) == 1 ? LMOE_W_DEPTH_FP8 : LMOE_W_DEPTH; }

// Per-workgroup context of the streaming kernel.
template <typename TOut, int NWB>
struct StreamCtx {
  BufRsrc a_rsrc, w_rsrc;
  uint32_t w_off[NWB];   // byte offset of this lane's part of its weight row, per n-block
  TOut* C;
  const float* sc;       // per-column scales of this group (fp8) or nullptr
  const int32_t* a_rows; // gather index (FC1) or nullptr (rows relative to the group)
  uint32_t a_row_bytes;  // lda * sizeof(TA)
  int64_t ldc;
  int K, N, gs, col0, wave, fr, fq, ac, ar0;
};

// One pass over up to 16 * NMB rows of a group: stream the group's weight
// tile through registers once, multiply with the staged token rows.
template <typename Mma, typename TA, typename TW, typename TOut, int MB_MAX, int NMB, int NWB,
          int WD, int ACT, bool SCALE>
__device__ __forceinline__ void stream_pass(const StreamCtx<TOut, NWB>& c, int p0, int rows,
                                            u32x4 (*As)[MB_MAX * 16 * kStageChunks]) {
  using Tr = StreamTraits<TA, TW>;
  constexpr int EPC = Tr::EPC;
  constexpr int KE = kStageChunks * EPC;    // reduction elements per stage
  constexpr int NS = KE / Tr::KSTEP;        // MFMA steps per stage (4)
  constexpr bool FP8 = sizeof(TW) == 1;
  constexpr int NLD = FP8 ? NS / 2 : NS;    // 16-byte weight loads per n-block per stage
  constexpr uint32_t W_STAGE_BYTES = KE * sizeof(TW);
  constexpr uint32_t A_STAGE_BYTES = KE * sizeof(TA);
  const int K = c.K;
  const int nst = (K + KE - 1) / KE;

  // byte offset of this thread's staged token rows (out of range = padding)
  uint32_t a_row_off[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i) {
    const int r = c.ar0 + 16 * i;
    if (r < rows) {
      const int row = c.a_rows ? c.a_rows[c.gs + p0 + r] : p0 + r;
      a_row_off[i] = static_cast<uint32_t>(row) * c.a_row_bytes + c.ac * 16u;
    } else {
      a_row_off[i] = kOutOfRange;
    }
  }

  f32x4_t acc[NMB][NWB];
#pragma unroll
  for (int i = 0; i < NMB; ++i)
#pragma unroll
    for (int j = 0; j < NWB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[2][NMB];
  u32x4 bw[WD + 1][NWB][NLD];

  // token chunk (row i, column ac) of stage st; past the end of K -> zero
#define LMOE_LOAD_A(st, ra)                                                                  \
  do {                                                                                       \
    const bool in_k_ = (st) * KE + c.ac * EPC < K;                                           \
    const uint32_t so_ = (st) * A_STAGE_BYTES;                                               \
    _Pragma("unroll") for (int i = 0; i < NMB; ++i)                                          \
      ra[i] = buffer_load_chunk(c.a_rsrc, in_k_ ? a_row_off[i] : kOutOfRange, so_);         \
  } while (0)
#define LMOE_STORE_A(buf, ra)                                                                \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < NMB; ++i) {                                        \
      const int r_ = c.ar0 + 16 * i;                                                         \
      As[buf][r_ * kStageChunks + (c.ac ^ (r_ & 15))] = ra[i];                               \
    }                                                                                        \
  } while (0)
  // weight chunk j of stage st for each n-block; the chunk's byte position
  // inside the stage is a compile-time constant folded into the instruction
#define LMOE_LOAD_W(st, br)                                                                  \
  do {                                                                                       \
    const bool live_ = (st) < nst;                                                           \
    const uint32_t so_ = (st) * W_STAGE_BYTES;                                               \
    _Pragma("unroll") for (int nb = 0; nb < NWB; ++nb) {                                     \
      const uint32_t vo_ = live_ ? c.w_off[nb] + so_ : kOutOfRange;                          \
      _Pragma("unroll") for (int j = 0; j < NLD; ++j)                                        \
        br[nb][j] = buffer_load_chunk<LMOE_W_CPOL>(c.w_rsrc, vo_ + 64u * j, 0u);            \
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
      const int c_ = Tr::elem_of(s, c.fq) / EPC;                                             \
      _Pragma("unroll") for (int mb = 0; mb < NMB; ++mb) {                                   \
        const int r_ = mb * 16 + c.fr;                                                       \
        const u32x4 af_ = As[buf][r_ * kStageChunks + (c_ ^ (r_ & 15))];                     \
        _Pragma("unroll") for (int nb = 0; nb < NWB; ++nb) Mma::mma(acc[mb][nb], af_, bfr[nb]); \
      }                                                                                      \
    }                                                                                        \
  } while (0)

  // Stage st is multiplied from register buffer bw[st % (WD+1)] and LDS
  // buffer st % 2.  Its weights were requested WD stages earlier; its token
  // rows two stages earlier (into register set ra[st % 2]) and written to LDS
  // one stage earlier, so neither latency sets the stage rate.  Every
  // prefetch is unconditional (past the end of K it reads zeros or is never
  // used) and is issued before the multiplies it overlaps.
  LMOE_LOAD_A(0, ra[0]);
#pragma unroll
  for (int i = 0; i < WD; ++i) LMOE_LOAD_W(i, bw[i]);
  LMOE_LOAD_A(1, ra[1]);
  LMOE_STORE_A(0, ra[0]);
  __syncthreads();
  // period of the register rotation: lcm(2, WD + 1) stages
  constexpr int P = (WD + 1) % 2 == 0 ? WD + 1 : 2 * (WD + 1);
  for (int st0 = 0; st0 < nst; st0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int st = st0 + u;
      if (st >= nst) break;
      LMOE_LOAD_W(st + WD, bw[(u + WD) % (WD + 1)]);
      LMOE_LOAD_A(st + 2, ra[u % 2]);
      __builtin_amdgcn_sched_barrier(0);
      LMOE_COMPUTE(u % 2, bw[u % (WD + 1)]);
      LMOE_STORE_A((u + 1) % 2, ra[(u + 1) % 2]);
      __syncthreads();
    }
  }
#undef LMOE_LOAD_A
#undef LMOE_STORE_A
#undef LMOE_LOAD_W
#undef LMOE_COMPUTE

  // Epilogue.  The accumulator holds C[4*fq + v][fr] of each 16x16 block, so
  // direct stores would be 2- or 4-byte pieces scattered over many rows.  The
  // tile goes through LDS instead (the token-row buffers are free after the
  // last barrier) and leaves as whole 16-byte chunks of contiguous row
  // segments.
  constexpr int NT = 4 * NWB * 16;            // columns of the workgroup tile
  constexpr int CPR = NT * sizeof(TOut) / 16; // 16-byte chunks per tile row
  static_assert(MB_MAX * 16 * NT * sizeof(TOut) <= sizeof(u32x4) * 2 * MB_MAX * 16 * kStageChunks,
                "output tile must fit the LDS staging buffers");
  TOut* Ct = reinterpret_cast<TOut*>(&As[0][0]);
#pragma unroll
  for (int nb = 0; nb < NWB; ++nb) {
    const int colt = c.wave * NWB * 16 + nb * 16 + c.fr;
    const int col = c.col0 + colt;
    const float s = (SCALE && col < c.N) ? c.sc[col] : 1.f;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float val = acc[mb][nb][v];
        if (SCALE) val *= s;
        store_elem<TOut>(Ct + (mb * 16 + c.fq * 4 + v) * NT + colt, apply_act<ACT>(val));
      }
    }
  }
  __syncthreads();
  const u32x4* Cv = reinterpret_cast<const u32x4*>(Ct);
  for (int q = c.wave * 64 + c.fq * 16 + c.fr; q < rows * CPR; q += 256) {
    const int r = q / CPR, ch = q % CPR;
    const int col = c.col0 + ch * (16 / static_cast<int>(sizeof(TOut)));
    if (col < c.N)  // N is a multiple of 16 elements: a chunk is all in or all out
      *reinterpret_cast<u32x4*>(c.C + (int64_t)(c.gs + p0 + r) * c.ldc + col) = Cv[q];
  }
}

// MB_MAX m-blocks of 16 rows per pass, NWB n-blocks of 16 weight rows per wave.
// One workgroup per work item (group, tile of NT columns); items are ordered
// so that each XCD receives one contiguous range of them.
template <typename Mma, typename TA, typename TW, typename TOut, int MB_MAX, int NWB, int ACT,
          bool SCALE>
#ifndef LMOE_STREAM_OCC
#define LMOE_STREAM_OCC 2
#endif
__global__ __launch_bounds__(256, MB_MAX * NWB <= 8 ? LMOE_STREAM_OCC : 1) void gemm_stream_kernel(GemmArgs p) {
  constexpr int MROWS = MB_MAX * 16;
  constexpr int NT = 4 * NWB * 16;          // output columns per work item
  __shared__ u32x4 As[2][MROWS * kStageChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n_tiles = (p.N + NT - 1) / NT;
  const int item = xcd_contiguous_item(blockIdx.x, gridDim.x, p.G * n_tiles);
  if (item < 0) return;
  const int g = item / n_tiles;
  const int gs = p.g_off[g];
  const int cnt = p.g_off[g + 1] - gs;
  if (cnt <= 0) return;

  StreamCtx<TOut, NWB> c;
  // token rows: the whole A for a gather, else the group's own rows
  const TA* abase = static_cast<const TA*>(p.A);
  if (!p.a_rows) abase += (int64_t)gs * p.lda;
  const uint64_t a_bytes = (uint64_t)(p.a_rows ? p.a_nrows : cnt) * p.lda * sizeof(TA);
  c.a_rsrc = make_rsrc(abase, a_bytes);
  const TW* wbase = static_cast<const TW*>(p.B) + (int64_t)g * p.b_gstride;
  c.w_rsrc = make_rsrc(wbase, (uint64_t)p.N * p.ldb * sizeof(TW));
  c.C = static_cast<TOut*>(p.C);
  c.sc = SCALE ? p.b_scale + (int64_t)g * p.s_gstride : nullptr;
  c.a_rows = p.a_rows;
  c.a_row_bytes = static_cast<uint32_t>(p.lda * sizeof(TA));
  c.ldc = p.ldc;
  c.K = p.K;
  c.N = p.N;
  c.gs = gs;
  c.col0 = (item % n_tiles) * NT;
  c.wave = wave;
  c.fr = lane & 15;
  c.fq = lane >> 4;
  c.ac = tid & 15;   // A staging: thread owns chunk column ac of rows ar0 + 16 i
  c.ar0 = tid >> 4;
  // byte position of this lane's first chunk in its weight row (lane group
  // fq supplies 16 bytes of every 64); rows past N read as zero
#pragma unroll
  for (int nb = 0; nb < NWB; ++nb) {
    const int n = c.col0 + wave * NWB * 16 + nb * 16 + c.fr;
    c.w_off[nb] = n < p.N ? static_cast<uint32_t>(n) * static_cast<uint32_t>(p.ldb * sizeof(TW)) +
                                16u * c.fq
                          : kOutOfRange;
  }

  for (int p0 = 0; p0 < cnt; p0 += MROWS) {
    const int rows = min(MROWS, cnt - p0);
    const int nmb = (rows + 15) >> 4;
#define LMOE_PASS(n) \
  stream_pass<Mma, TA, TW, TOut, MB_MAX, n, NWB, stream_w_depth<TW>(), ACT, SCALE>(c, p0, rows, As)
    if constexpr (MB_MAX == 4) {
      switch (nmb) {
        case 1: LMOE_PASS(1); break;
        case 2: LMOE_PASS(2); break;
        case 3: LMOE_PASS(3); break;
        default: LMOE_PASS(4); break;
      }
    } else {
      switch (nmb) {
        case 1: LMOE_PASS(1); break;
        case 2: LMOE_PASS(2); break;
        case 3: LMOE_PASS(3); break;
        case 4: LMOE_PASS(4); break;
        case 5: LMOE_PASS(5); break;
        case 6: LMOE_PASS(6); break;
        case 7: LMOE_PASS(7); break;
        default: LMOE_PASS(8); break;
      }
    }
#undef LMOE_PASS
    __syncthreads();  // the next pass restages the LDS buffers
  }
}

// n-blocks of 16 weight rows per wave: two with up to 64 rows per pass, one
// with 128 (the accumulators of the larger pass then leave room for two
// workgroups per compute unit)
#ifndef LMOE_STREAM_NWB
#define LMOE_STREAM_NWB 2
#endif
#ifndef LMOE_STREAM_NWB_MB8
#define LMOE_STREAM_NWB_MB8 1
#endif

template <typename Mma, typename TA, typename TW, typename TOut, int MB>
hipError_t launch_s(const GemmArgs& a, hipStream_t s) {
  constexpr int NWB = MB >= 8 ? LMOE_STREAM_NWB_MB8 : LMOE_STREAM_NWB;
  constexpr int NT = 4 * NWB * 16;
  const int64_t n_tiles = (a.N + NT - 1) / NT;
  const int64_t total = n_tiles * a.G;
  const int64_t grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  // the epilogue stores whole 16-byte chunks: output width and stride are
  // multiples of 16 elements (true of the expert widths m and l)
  if (a.N % 16 || a.ldc % 16) return hipErrorInvalidValue;
  // 32-bit buffer offsets: token rows and one expert matrix stay below 2 GiB
  const uint64_t a_rows = a.a_rows ? (uint64_t)a.a_nrows : (uint64_t)a.max_rows;
  if (a_rows * a.lda * sizeof(TA) >= (1ull << 31) ||
      (uint64_t)a.N * a.ldb * sizeof(TW) >= (1ull << 31))
    return hipErrorInvalidValue;
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
