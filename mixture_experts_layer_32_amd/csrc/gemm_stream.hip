// Weight-streaming grouped GEMM for the latent experts when each expert
// receives few token copies (decode regime), for gfx950.
//
// C[r][n] = act(scale[g][n] * sum_k A[arow(r)][k] * W[g][n][k]),  r in group g
// (SwiGLU: W's rows are (up, gate) pairs and C[r][i] = up_i * SiLU(gate_i))
//
// With a few dozen rows per expert the GEMM is bound by reading the expert
// weights from HBM once, so the kernel is built around that stream:
//  - A work unit is (expert, tile of 64 * NWB output columns, pass of up to
//    16 * MB_MAX rows).  The grid is persistent: as many workgroups as stay
//    resident, each XCD owning one contiguous range of units, so the tiles
//    of one expert run on one XCD and share its token rows in that XCD's L2.
//  - The weight stream of a workgroup does not stop between units.  While a
//    unit streams, the next unit's group bounds and gather indices are read,
//    and its first weight and token stages are requested during the unit's
//    last stages.  Under a saturated memory queue each of those dependent
//    reads costs microseconds, which a workgroup per unit would spend
//    without weight bytes in flight.
//  - Barriers order LDS only (an LDS-scoped fence around s_barrier): the
//    epilogue's stores and the prefetches stay in flight across them.
//  - Each wave streams its own 16 * NWB weight rows straight from global
//    memory into registers in the MFMA B-operand layout with raw buffer
//    loads: 4 lanes per weight row side by side, so one load instruction
//    reads 64 contiguous bytes of each of 16 rows.  WD stages of weights are
//    in flight while the current one is multiplied.
//  - The token rows of a unit are staged through LDS per K stage
//    (double-buffered, two stages ahead), gathered through token_of for FC1:
//    this is the dispatch of the token copies, done without materialising
//    them.
//  - fp8 (OCP E4M3) weights are widened to bf16 in registers (exact) and the
//    per-row scale is applied to the fp32 accumulator in the epilogue.
// Experts with more rows than one pass holds take several passes (units);
// the weights are then streamed once per pass.
//
// Out-of-range buffer offsets read as zero without a memory request: padding
// token rows, token chunks past the end of K, stages past the end of K and
// prefetches past the last unit use that, so no select on loaded data delays
// a wait.  Weight chunks past the end of K inside the last stage (K not a
// multiple of the stage) read the next weight row or zero; they meet zero
// token values.  Every offset is carried in the per-lane offset, which is
// what the range check applies to.
#include <algorithm>
#include <type_traits>

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
template <> struct StreamTraits<uint16_t, fp4x2_t> {   // bf16 tokens, MXFP4 weights: a
  static constexpr int EPC = 8;                         // lane owns the 32 consecutive
  static constexpr int KSTEP = 32;                      // indices of one 16-byte chunk (one
  __device__ __forceinline__ static int elem_of(int s, int q) {  // scale block), used by the
    return 32 * q + 8 * s;                              // stage's 4 steps
  }
};
template <> struct StreamTraits<float, float> {        // fp32 tokens and weights
  static constexpr int EPC = 4;
  static constexpr int KSTEP = 16;
  __device__ __forceinline__ static int elem_of(int s, int q) { return 16 * s + 4 * q; }
};


constexpr int kStageChunks = 16;  // 16-byte chunks of A per row per K stage (256 bytes)

// Stage geometry of one (token type, weight type) pair.
template <typename TA, typename TW>
struct StreamShape {
  using Tr = StreamTraits<TA, TW>;
  static constexpr int EPC = Tr::EPC;
  static constexpr int KE = kStageChunks * EPC;    // reduction elements per stage
  static constexpr int NS = KE / Tr::KSTEP;        // MFMA steps per stage (4)
  static constexpr bool FP8 = std::is_same_v<TW, uint8_t>;
  static constexpr bool FP4 = std::is_same_v<TW, fp4x2_t>;
  // 16-byte weight loads per n-block per stage
  static constexpr int NLD = FP8 ? NS / 2 : FP4 ? NS / 4 : NS;
  static constexpr uint32_t W_STAGE_BYTES = FP4 ? KE / 2 : KE * sizeof(TW);
  static constexpr uint32_t A_STAGE_BYTES = KE * sizeof(TA);
  // K stages of weights requested ahead of the one being multiplied.  An fp8
  // stage is half the bytes of a bf16 one and its registers a quarter (one
  // n-block), so fp8 (and fp4) look further ahead.
  static constexpr int WD = (FP8 || FP4) ? 3 : 1;
  // Register sets rotate: weights modulo WD + 1 stages, token rows modulo 2.
  // Units are padded to a multiple of this period, so every unit starts at
  // rotation phase 0 and the rotation stays in compile-time indices.
  static constexpr int P = (WD + 1) % 2 == 0 ? WD + 1 : 2 * (WD + 1);
};

// One work unit.  The scalars are wave-uniform; the offsets are per lane.
template <int MB_MAX, int NWB>
struct Unit {
  int local;         // position in the workgroup's item sequence
  int g, col0;       // group (expert) and first output column
  int gs, cnt;       // the group's first row and row count
  int p0, rows;      // this pass's first row (within the group) and rows (0: none)
  int valid;          // 0: past the end of the sequence (nothing to load or store)
  BufRsrc w_rsrc;            // the group's weight matrix
  uint32_t w_off[NWB];       // byte offset of this lane's chunk in its weight row, per n-block
  BufRsrc s_rsrc;            // MXFP4: the group's block scales
  uint32_t s_off[NWB];       // MXFP4: this lane's scale byte at stage 0, per n-block
  uint32_t a_off[MB_MAX];    // byte offset of this thread's chunk column in token row ar0 + 16 i

  // field by field, so that the compiler keeps every field in registers
  __device__ __forceinline__ void assign(const Unit& o) {
    local = o.local;
    g = o.g;
    col0 = o.col0;
    gs = o.gs;
    cnt = o.cnt;
    p0 = o.p0;
    rows = o.rows;
    valid = o.valid;
    w_rsrc = o.w_rsrc;
    s_rsrc = o.s_rsrc;
#pragma unroll
    for (int i = 0; i < NWB; ++i) w_off[i] = o.w_off[i];
#pragma unroll
    for (int i = 0; i < NWB; ++i) s_off[i] = o.s_off[i];
#pragma unroll
    for (int i = 0; i < MB_MAX; ++i) a_off[i] = o.a_off[i];
  }
};

constexpr int kStreamOcc = 2;  // resident workgroups per compute unit

// MB_MAX m-blocks of 16 rows per pass, NWB n-blocks of 16 weight rows per
// wave, 4 waves.
template <typename Mma, typename TA, typename TW, typename TOut, int MB_MAX, int NWB, int ACT,
          bool SCALE>
__global__ __launch_bounds__(256, kStreamOcc) void gemm_stream_kernel(GemmArgs p) {
  using S = StreamShape<TA, TW>;
  using Tr = typename S::Tr;
  using U = Unit<MB_MAX, NWB>;
  constexpr int MROWS = MB_MAX * 16;
  constexpr int NT = 4 * NWB * 16;                    // output columns per unit
  constexpr int WD = S::WD, P = S::P, NLD = S::NLD, NS = S::NS, KE = S::KE, EPC = S::EPC;
  // SwiGLU: weight-row pairs (up, gate) give one output column each
  constexpr bool GLU = ACT == kActSwiGlu;
  constexpr int NTO = GLU ? NT / 2 : NT;               // output columns per unit
  constexpr int CPR = NTO * static_cast<int>(sizeof(TOut)) / 16;  // 16-byte chunks per tile row
  __shared__ u32x4 As[2][MROWS * kStageChunks];
  __shared__ u32x4 Cs[MROWS * CPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fq = lane >> 4;
  const int ac = tid & 15, ar0 = tid >> 4;  // A staging: chunk column ac of rows ar0 + 16 i
  const int n_tiles = (p.N + NT - 1) / NT;
  // groups visited: all, or (sparse batches) the listed ones with rows
  const int g_count = p.g_active ? __builtin_amdgcn_readfirstlane(p.g_tiles[p.G]) : p.G;
  const int total = g_count * n_tiles;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int slots = gridDim.x / kNumXcd;
  const int item_base = (blockIdx.x % kNumXcd) * per_xcd;
  const int K = p.K;
  const int nst = (K + KE - 1) / KE;
  const int nsp = (nst + P - 1) / P * P;  // stages per unit, padded to the rotation period
  const int s_take = min(1, nsp - 2);     // stage at which the next unit's bounds are used
  const BufRsrc a_rsrc =
      make_rsrc(p.A, (uint64_t)(p.a_rows ? p.a_nrows : p.max_rows) * p.lda * sizeof(TA));
  const BufRsrc goff_rsrc = make_rsrc(p.g_off, (uint64_t)(p.G + 1) * sizeof(int32_t));
  const uint32_t a_row_bytes = static_cast<uint32_t>(p.lda * sizeof(TA));
  const uint32_t w_row_bytes = static_cast<uint32_t>(p.ldb * sizeof(TW));
  const TW* const wglob = static_cast<const TW*>(p.B);
  TOut* const C = static_cast<TOut*>(p.C);

  // ---- unit bookkeeping
  // identity of the first pass of the item at sequence position `local`
  auto set_item = [&](U& u, int local) {
    const int item = item_base + local;
    u.local = local;
    u.valid = local < per_xcd && item < total;
    const int it = u.valid ? item : 0;
    u.g = it / n_tiles;
    if (p.g_active && u.valid) u.g = __builtin_amdgcn_readfirstlane(p.g_active[u.g]);
    u.col0 = (it % n_tiles) * NT;
    u.p0 = 0;
    u.gs = 0;
    u.cnt = 0;
    u.rows = 0;
    u.w_rsrc = make_rsrc(wglob + (int64_t)u.g * p.b_gstride, (uint64_t)p.N * w_row_bytes);
    if constexpr (S::FP4)
      u.s_rsrc = make_rsrc(p.b_mx + (int64_t)u.g * p.mx_gstride, (uint64_t)p.N * p.mx_ld);
#pragma unroll
    for (int nb = 0; nb < NWB; ++nb) {
      const int n = u.col0 + wave * NWB * 16 + nb * 16 + fr;
      u.w_off[nb] = (u.valid && n < p.N) ? static_cast<uint32_t>(n) * w_row_bytes + 16u * fq
                                         : kOutOfRange;
      // the lane's chunk of stage s is block 4 s + fq of its row
      if constexpr (S::FP4)
        u.s_off[nb] = (u.valid && n < p.N) ? static_cast<uint32_t>(n * p.mx_ld) + fq : kOutOfRange;
    }
  };
  // group bounds g_off[g], g_off[g + 1]: a vector load, so that waiting for
  // it is ordered with the stream's own loads instead of the LDS counter
  u32x2 bounds = u32x2{0u, 0u};
  auto issue_bounds = [&](const U& u) {
    bounds = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                   goff_rsrc, static_cast<int>(u.valid ? u.g * 4u : kOutOfRange), 0, 0));
  };
  auto take_bounds = [&](U& u) {
    const int gs = __builtin_amdgcn_readfirstlane(static_cast<int>(bounds.x));
    const int ge = __builtin_amdgcn_readfirstlane(static_cast<int>(bounds.y));
    u.gs = gs;
    u.cnt = u.valid ? ge - gs : 0;
    u.rows = max(0, min(MROWS, u.cnt - u.p0));
  };
  // token row of each staged row (FC1 gathers it through a_rows)
  int tok[MB_MAX];
  auto issue_rows = [&](const U& u) {
#pragma unroll
    for (int i = 0; i < MB_MAX; ++i) {
      const int r = ar0 + 16 * i;
      const int lr = u.gs + u.p0 + r;
      tok[i] = (p.a_rows && r < u.rows) ? p.a_rows[lr] : lr;
    }
  };
  auto take_rows = [&](U& u) {
#pragma unroll
    for (int i = 0; i < MB_MAX; ++i) {
      const int r = ar0 + 16 * i;
      u.a_off[i] = r < u.rows ? static_cast<uint32_t>(tok[i]) * a_row_bytes + 16u * ac : kOutOfRange;
    }
  };

  // ---- loads of one stage
  // weight chunks of stage s; the chunk's position inside the stage is a
  // compile-time constant
  auto load_w = [&](const U& u, int s, bool live, u32x4 (&br)[NWB][NLD], uint32_t (&bs)[NWB]) {
    const uint32_t so = static_cast<uint32_t>(s) * S::W_STAGE_BYTES;
#pragma unroll
    for (int nb = 0; nb < NWB; ++nb) {
      const uint32_t vo = live ? u.w_off[nb] + so : kOutOfRange;
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        br[nb][j] = buffer_load_chunk<kCpolDefault>(u.w_rsrc, vo + 64u * j, 0u);
      if constexpr (S::FP4)
        bs[nb] = buffer_load_byte(u.s_rsrc, live ? u.s_off[nb] + 4u * s : kOutOfRange);
    }
  };
  // token chunk (row ar0 + 16 i, column ac) of stage s; past K -> zero
  auto load_a = [&](const U& u, int s, u32x4 (&ra)[MB_MAX]) {
    const bool in_k = s * KE + ac * EPC < K;
    const uint32_t so = static_cast<uint32_t>(s) * S::A_STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < MB_MAX; ++i)
      ra[i] = buffer_load_chunk(a_rsrc, in_k ? u.a_off[i] + so : kOutOfRange, 0u);
  };
  auto store_a = [&](int buf, const u32x4 (&ra)[MB_MAX]) {
#pragma unroll
    for (int i = 0; i < MB_MAX; ++i) {
      const int r = ar0 + 16 * i;
      As[buf][r * kStageChunks + (ac ^ (r & 15))] = ra[i];
    }
  };

  f32x4_t acc[MB_MAX][NWB];
#pragma unroll
  for (int i = 0; i < MB_MAX; ++i)
#pragma unroll
    for (int j = 0; j < NWB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, const u32x4 (&br)[NWB][NLD], const uint32_t (&bs)[NWB]) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 bfr[NWB];
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb) {
        if constexpr (S::FP4) {
          // dword s of the lane's chunk: elements 32 fq + 8 s .. + 7
          bfr[nb] = fp4x8_to_bf16x8(br[nb][0][s], e8m0_to_f32(bs[nb]));
        } else if constexpr (S::FP8) {
          u32x4 lo, hi;
          fp8_chunk_to_bf16(br[nb][s >> 1], lo, hi);
          bfr[nb] = (s & 1) ? hi : lo;
        } else {
          bfr[nb] = br[nb][s];
        }
      }
      const int c = Tr::elem_of(s, fq) / EPC;
#pragma unroll
      for (int mb = 0; mb < MB_MAX; ++mb) {
        const int r = mb * 16 + fr;
        const u32x4 af = As[buf][r * kStageChunks + (c ^ (r & 15))];
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb) Mma::mma(acc[mb][nb], af, bfr[nb]);
      }
    }
  };

  // ---- first unit: its weights depend on the item alone and are requested
  // before the dependent reads of its bounds, gather indices and token rows
  U cur, nxt;
  set_item(cur, blockIdx.x / kNumXcd);
  if (!cur.valid) return;
  u32x4 bw[WD + 1][NWB][NLD];
  uint32_t bsw[WD + 1][NWB];  // MXFP4 block scales of each weight stage
  u32x4 ra[2][MB_MAX];
#pragma unroll
  for (int i = 0; i < WD; ++i) load_w(cur, i, i < nst, bw[i], bsw[i]);
  issue_bounds(cur);
  take_bounds(cur);
  issue_rows(cur);
  take_rows(cur);
  load_a(cur, 0, ra[0]);
  load_a(cur, 1, ra[1]);
  store_a(0, ra[0]);
  lds_barrier();
  nxt.assign(cur);

  // Stage st of a unit is multiplied from register set bw[st % (WD+1)] and
  // LDS buffer st % 2.  Its weights were requested WD stages earlier, its
  // token rows two stages earlier (into ra[st % 2]) and written to LDS one
  // stage earlier.  Requests past the unit's last stage go to the next unit.
  for (;;) {
    for (int st0 = 0; st0 < nsp; st0 += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int st = st0 + u;
        // the next unit: identity and bounds request, then bounds and gather
        // indices, then its token-row offsets, each a stage or more apart
        if (st == 0) {
          if (cur.p0 + MROWS < cur.cnt) {  // another pass over the same group
            nxt.assign(cur);
            nxt.p0 = cur.p0 + MROWS;
            nxt.rows = min(MROWS, cur.cnt - nxt.p0);
          } else {
            set_item(nxt, cur.local + slots);
            issue_bounds(nxt);
          }
        }
        if (st == s_take) {
          if (nxt.p0 == 0) take_bounds(nxt);
          issue_rows(nxt);
        }
        if (st == nsp - 2) take_rows(nxt);
        // weights of stage st + WD, token rows of stage st + 2
        const int sw = st + WD;
        if (sw < nsp)
          load_w(cur, sw, sw < nst && cur.rows > 0, bw[(u + WD) % (WD + 1)], bsw[(u + WD) % (WD + 1)]);
        else
          load_w(nxt, sw - nsp, sw - nsp < nst && nxt.rows > 0, bw[(u + WD) % (WD + 1)],
                 bsw[(u + WD) % (WD + 1)]);
        const int sa = st + 2;
        if (sa < nsp) load_a(cur, sa, ra[u % 2]);
        else load_a(nxt, sa - nsp, ra[u % 2]);
        __builtin_amdgcn_sched_barrier(0);
        compute(u % 2, bw[u % (WD + 1)], bsw[u % (WD + 1)]);
        store_a((u + 1) % 2, ra[(u + 1) % 2]);
        lds_barrier();
      }
    }

    // Epilogue.  The accumulator holds C[4*fq + v][fr] of each 16x16 block,
    // so direct stores would be 2- or 4-byte pieces scattered over many
    // rows.  The tile goes through LDS and leaves as whole 16-byte chunks
    // of contiguous row segments; the stores overlap the next unit.
    if (cur.rows > 0) {
      TOut* Ct = reinterpret_cast<TOut*>(&Cs[0]);
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb) {
        const int colt = wave * NWB * 16 + nb * 16 + fr;
        const int col = cur.col0 + colt;
        const float sc = (SCALE && col < p.N) ? p.b_scale[(int64_t)cur.g * p.s_gstride + col] : 1.f;
#pragma unroll
        for (int mb = 0; mb < MB_MAX; ++mb) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float val = acc[mb][nb][v];
            if (SCALE) val *= sc;
            if constexpr (GLU) {
              // a lane holds one column: the gate of an even (up) column is
              // in the next lane, which holds the odd column
              const float gate = __shfl_xor(val, 1);
              if ((fr & 1) == 0)
                store_elem<TOut>(Ct + (mb * 16 + fq * 4 + v) * NTO + colt / 2, swiglu(val, gate));
            } else {
              store_elem<TOut>(Ct + (mb * 16 + fq * 4 + v) * NT + colt, apply_act<ACT>(val));
            }
          }
        }
      }
      lds_barrier();
      const int64_t row0 = (int64_t)cur.gs + cur.p0;
      const int n_out = GLU ? p.N / 2 : p.N;
      const int col0_out = GLU ? cur.col0 / 2 : cur.col0;
      for (int q = tid; q < cur.rows * CPR; q += 256) {
        const int r = q / CPR, ch = q % CPR;
        const int col = col0_out + ch * (16 / static_cast<int>(sizeof(TOut)));
        if (col < n_out)  // the output width is a multiple of 16 elements: a chunk is all in or all out
          *reinterpret_cast<u32x4*>(C + (row0 + r) * p.ldc + col) = Cs[q];
      }
    }
#pragma unroll
    for (int i = 0; i < MB_MAX; ++i)
#pragma unroll
      for (int j = 0; j < NWB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (!nxt.valid) break;
    cur.assign(nxt);
  }
}

template <typename Mma, typename TA, typename TW, typename TOut, int MB>
hipError_t launch_s(const GemmArgs& a, hipStream_t s) {
  // n-blocks of 16 weight rows per wave: two with up to 64 rows per pass,
  // one with 128 (the accumulators of the larger pass then leave room for
  // two workgroups per compute unit); the same for every weight type
  constexpr int NWB = MB >= 8 ? 1 : 2;
  constexpr int NT = 4 * NWB * 16;
  if (a.g_off == nullptr || a.G < 1 || (a.g_active && !a.g_tiles)) return hipErrorInvalidValue;
  const int64_t n_tiles = (a.N + NT - 1) / NT;
  const int64_t total = n_tiles * a.G;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  // the epilogue stores whole 16-byte chunks: output width and stride are
  // multiples of 16 elements (true of the expert widths m and l)
  if (a.N % 16 || a.ldc % 16) return hipErrorInvalidValue;
  if (a.act == kActSwiGlu && (a.N % 32 || a.ldc < a.N / 2)) return hipErrorInvalidValue;
  // 32-bit buffer offsets: token rows and one expert matrix stay below 2 GiB
  const uint64_t a_rows = a.a_rows ? (uint64_t)a.a_nrows : (uint64_t)a.max_rows;
  if (a_rows * a.lda * sizeof(TA) >= (1ull << 31) ||
      (uint64_t)a.N * a.ldb * sizeof(TW) >= (1ull << 31))
    return hipErrorInvalidValue;
  // persistent grid: the resident workgroups, a multiple of the XCD count,
  // no more per XCD than it has work items
  const int64_t per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int64_t slots = std::max<int64_t>(1, (int64_t)kStreamOcc * device_compute_units() / kNumXcd);
  const int64_t grid = std::min(per_xcd, slots) * kNumXcd;
  const bool scale = a.b_scale != nullptr;
  if (a.act == kActSqRelu) {
    if (scale) gemm_stream_kernel<Mma, TA, TW, TOut, MB, NWB, kActSqRelu, true><<<dim3(grid), dim3(256), 0, s>>>(a);
    else gemm_stream_kernel<Mma, TA, TW, TOut, MB, NWB, kActSqRelu, false><<<dim3(grid), dim3(256), 0, s>>>(a);
  } else if (a.act == kActSwiGlu) {
    if (scale) gemm_stream_kernel<Mma, TA, TW, TOut, MB, NWB, kActSwiGlu, true><<<dim3(grid), dim3(256), 0, s>>>(a);
    else gemm_stream_kernel<Mma, TA, TW, TOut, MB, NWB, kActSwiGlu, false><<<dim3(grid), dim3(256), 0, s>>>(a);
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
  if (w_dt == Dt::MXFP4) {
    // whole scale blocks per row; one scale byte per block
    if (!a.b_mx || a.K % 32 || a.mx_ld < a.K / 32 || a.ldb < a.K / 2 ||
        (uint64_t)a.N * a.mx_ld >= (1ull << 31))
      return hipErrorInvalidValue;
    return launch_s<MmaBf16, uint16_t, fp4x2_t, uint16_t, MB>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int device_compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

hipError_t launch_gemm_stream(const GemmArgs& a, Dt a_dt, Dt w_dt, Dt out_dt, int mb_max,
                              hipStream_t s) {
  if (mb_max <= 4) return launch_mb<4>(a, a_dt, w_dt, out_dt, s);
  return launch_mb<8>(a, a_dt, w_dt, out_dt, s);
}

}  // namespace lmoe
