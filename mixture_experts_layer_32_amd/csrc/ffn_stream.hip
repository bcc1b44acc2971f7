// Fused latent expert FFN for the decode regime, for gfx950:
//
//   H = sqrelu(A_g W1_g^T)   rows of expert g  x  m   (kept in LDS, bf16)
//   Y = H W2_g^T             rows of expert g  x  l   (written to HBM, bf16)
//
// (the expert FFN of the LatentMoE paper, Eq. (2): both expert GEMMs run in
// the latent width l, with the squared-ReLU activation of Table 2).  With
// SwiGLU experts W1 holds 2m rows, up-projection and gate rows interleaved,
// and H[i] = up_i * SiLU(gate_i): FC1 streams twice the rows.  With MXFP4
// weights (E2M1 pairs, an E8M0 scale per 32 elements) a lane loads 32
// consecutive elements of a row (16 bytes, one scale block, and that
// block's scale byte) for two stages, a double stage of 128 elements, and
// widens 16 of them per stage to two bf16 MFMA operands; the staged token
// chunks and the H fragments take the matching reduction indices.  (One
// 8-byte piece per stage, half as many bytes per request, ran 1.4x slower.)
//
// With a few dozen token rows per expert both GEMMs are bound by streaming
// the expert weights from HBM.  Writing H out and reading it back, as two
// separate kernels must, puts a write stream next to the weight reads, and
// on this part interleaved writes cost far more read bandwidth than their
// bytes.  Here one workgroup (8 waves) takes a whole expert: it computes H
// tile by tile into LDS, then streams W2 against H, so H never leaves the
// chip and the only writes are Y.
//  - One resident workgroup per compute unit (H of 48 rows x m <= 1536
//    fills the LDS); experts blockIdx.x, blockIdx.x + gridDim.x, ...
//  - A stage is 64 reduction elements.  Each wave streams 16 * NWB weight
//    rows into registers in the MFMA operand layout, 4 lanes side by side on
//    64 contiguous bytes of a row, WD stages ahead of the one multiplied
//    (MXFP4: two double stages ahead).
//  - One buffer resource per weight array (all experts) and 32-bit offsets:
//    per-expert resources for the current and the next unit overflowed the
//    scalar registers into lanes of a vector register.
//  - FC1's token rows are gathered through token_of and staged through LDS
//    two stages ahead (double-buffered, one barrier per FC1 stage).  FC2's
//    operand is H itself: the waves run through FC2 without barriers until
//    its last stage, after which the next expert's first token stage is
//    read.  (Reading the token fragments straight from L2 into every wave,
//    which needs no FC1 barriers, measured slower.)
//  - The weight stream does not stop at tile, GEMM or expert boundaries:
//    the next stage may belong to the next tile, to W2, or to the next
//    expert, whose group bounds and gather indices are read during the
//    current expert's first stages.
//  - Blocks are computed transposed (weights as the first MFMA operand), so
//    a lane holds 4 consecutive output columns of one row: H goes to LDS
//    and Y to HBM as 8-byte pieces.
// Out-of-range buffer offsets read zero without a memory request (padding
// rows, chunks past K, loads past the last expert); tiles are padded to a
// multiple of the register-rotation period with stages that load nothing.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMB = 3;                         // 16-row blocks of token rows per pass
constexpr int kRows = 16 * kMB;                // token rows per pass
constexpr int kNWB = 4;             // 16-row weight blocks per wave
constexpr int kTileN = kWaves * kNWB * 16;     // output columns per tile
constexpr int kKE = 64;                        // reduction elements per stage
constexpr int kNS = kKE / 32;                  // MFMA k-steps per stage
constexpr int kNLD = kNS;                      // 16-byte weight loads per n-block per stage
constexpr int kWD = 3;               // weight stages in flight ahead
// registers rotate: weights modulo kWD + 1 stages, staged token rows modulo 2
constexpr int kP = (kWD + 1) % 2 == 0 ? kWD + 1 : 2 * (kWD + 1);
// MXFP4: a lane's 16-byte weight piece is 32 elements (one scale block) and
// serves two stages (a double stage); weights run two double stages ahead
// in four register sets
constexpr int kWD4 = 4;
constexpr int kP4 = 8;
constexpr int kMaxM = 1536;                    // hidden width that fits in LDS
constexpr int kAChunks = kRows * (kKE / 8);    // staged token chunks per stage (384)

struct FfnUnit {
  int e;             // expert (group)
  int valid;         // 0: past the last expert
  int gs, cnt;       // first grouped row of the expert and its row count
  int p0, rows;      // this pass's first row (within the expert) and its rows
  uint32_t a_off;    // this thread's staged token chunk, or out of range

  __device__ __forceinline__ void assign(const FfnUnit& o) {
    e = o.e;
    valid = o.valid;
    gs = o.gs;
    cnt = o.cnt;
    p0 = o.p0;
    rows = o.rows;
    a_off = o.a_off;
  }
};

// Weight registers of one stage: bf16 rows (kNLD 16-byte chunks per n-block),
// or of one MXFP4 double stage (a 16-byte piece per n-block; the scales
// come in groups of four double stages, see load_sg)
struct WStageBf16 {
  u32x4 b[kNWB][kNLD];
};
struct WStageFp4 {
  u32x4 b[kNWB];
};

template <bool GLU, bool FP4>
__global__ __launch_bounds__(kThreads, 1) void ffn_stream_kernel(FfnArgs p) {
  using WS = std::conditional_t<FP4, WStageFp4, WStageBf16>;
  constexpr int KWD = FP4 ? kWD4 : kWD;      // weight stages in flight ahead
  constexpr int KP = FP4 ? kP4 : kP;         // unrolled stages (register rotation period)
  constexpr int NSLOT = FP4 ? 4 : kWD + 1;   // weight register sets
  __shared__ u32x4 Hs[kRows * kMaxM / 8];  // H, 16-byte chunk c of row r at c ^ (r & 7)
  __shared__ u32x4 As[2][kAChunks];        // FC1 token stages, chunk c of row r at c ^ ((r >> 1) & 7)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fq = lane >> 4;
  const int L = p.l, M = p.m;
  const int N1 = GLU ? 2 * M : M;            // FC1 weight rows (H columns x 2 with SwiGLU)
  // H row length: m rounded up to a stage (MXFP4: to a double stage)
  constexpr int kRound = FP4 ? 2 * kKE : kKE;
  const int mh = (M + kRound - 1) / kRound * kRound;
  const int hcpr = mh / 8;                   // 16-byte chunks per H row
  const int s1 = (L + kRound - 1) / kRound * (kRound / kKE);  // FC1 stages (reduction over l)
  const int s2 = mh / kKE;                   // FC2 stages (reduction over m)
  const int s1p = (s1 + KP - 1) / KP * KP;
  const int s2p = (s2 + KP - 1) / KP * KP;
  const int t1 = (N1 + kTileN - 1) / kTileN; // FC1 tiles (of W1 rows)
  const int t2 = (L + kTileN - 1) / kTileN;  // FC2 tiles (Y columns)
  const uint32_t rb1 = FP4 ? static_cast<uint32_t>(L) / 2u : static_cast<uint32_t>(L) * 2u;  // W1 row bytes
  const uint32_t rb2 = FP4 ? static_cast<uint32_t>(M) / 2u : static_cast<uint32_t>(M) * 2u;  // W2 row bytes
  const uint32_t sb1 = static_cast<uint32_t>(L) / 32u;  // MXFP4: scale bytes per W1 row
  const uint32_t sb2 = static_cast<uint32_t>(M) / 32u;  // and per W2 row
  const uint32_t a_row_bytes = static_cast<uint32_t>(p.lda) * 2u;
  const BufRsrc a_rsrc = make_rsrc(p.A, (uint64_t)p.a_nrows * p.lda * 2u);
  const BufRsrc goff_rsrc = make_rsrc(p.g_off, (uint64_t)(p.G + 1) * sizeof(int32_t));
  // one resource per weight (and scale) array, all experts; an expert's
  // matrix starts at e times its size (the launch keeps every array below
  // 2 GiB, so offsets stay 32-bit and below kOutOfRange)
  const uint32_t wm1 = static_cast<uint32_t>(N1) * rb1;   // bytes of one W1 matrix
  const uint32_t wm2 = static_cast<uint32_t>(L) * rb2;
  const uint32_t sm1 = static_cast<uint32_t>(N1) * sb1;   // MXFP4: bytes of its scales
  const uint32_t sm2 = static_cast<uint32_t>(L) * sb2;
  const BufRsrc w1r = make_rsrc(p.W1, (uint64_t)p.G * wm1);
  const BufRsrc w2r = make_rsrc(p.W2, (uint64_t)p.G * wm2);
  const BufRsrc s1r = make_rsrc(p.W1_mx, FP4 ? (uint64_t)p.G * sm1 : 0u);
  const BufRsrc s2r = make_rsrc(p.W2_mx, FP4 ? (uint64_t)p.G * sm2 : 0u);
  uint16_t* const Y = static_cast<uint16_t*>(p.Y);
  const int nl = wave * (kNWB * 16) + fr;    // weight row of n-block 0 within a tile
  const int ar = tid >> 3, ac = tid & 7;     // staged token chunk of this thread
  const bool a_thread = tid < kAChunks;

  // ---- unit bookkeeping
  auto set_expert = [&](FfnUnit& u, int e) {
    u.e = e;
    u.valid = e < p.G;
    u.gs = 0;
    u.cnt = 0;
    u.p0 = 0;
    u.rows = 0;
    u.a_off = kOutOfRange;
  };
  u32x2 bounds = u32x2{0u, 0u};
  auto issue_bounds = [&](const FfnUnit& u) {
    bounds = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                   goff_rsrc, static_cast<int>(u.valid ? u.e * 4u : kOutOfRange), 0, 0));
  };
  auto take_bounds = [&](FfnUnit& u) {
    const int gs = __builtin_amdgcn_readfirstlane(static_cast<int>(bounds.x));
    const int ge = __builtin_amdgcn_readfirstlane(static_cast<int>(bounds.y));
    u.gs = gs;
    u.cnt = u.valid ? ge - gs : 0;
    u.rows = min(kRows, u.cnt - u.p0);
  };
  // the next expert of this workgroup with rows (blocking reads; experts
  // without rows are rare in the decode regime)
  auto find_rows = [&](FfnUnit& u) {
    while (u.valid && u.cnt <= 0) {
      set_expert(u, u.e + gridDim.x);
      issue_bounds(u);
      take_bounds(u);
    }
  };
  int tok = 0;
  auto issue_rows = [&](const FfnUnit& u) {
    tok = (a_thread && ar < u.rows) ? p.a_rows[u.gs + u.p0 + ar] : 0;
  };
  // a thread's staged chunk ac of a stage: chunk ac of its 64 elements, or
  // with MXFP4 (a double stage covers 128 elements, lane fq of an n-block
  // holds elements 32 fq .. 32 fq + 31 of it, 16 per stage) chunk
  // 4 (ac / 2) + ac % 2 of the double stage, plus 2 in its second stage
  const uint32_t a_chunk = FP4 ? 4u * (ac >> 1) + (ac & 1) : static_cast<uint32_t>(ac);
  auto take_rows = [&](FfnUnit& u) {
    u.a_off = (a_thread && ar < u.rows) ? static_cast<uint32_t>(tok) * a_row_bytes + 16u * a_chunk
                                        : kOutOfRange;
  };

  // ---- stage positions: (gemm ph, tile t, stage ks); advance by d < kP
  // stages, possibly into the next unit
  auto advance = [&](int ph, int t, int ks, int d, int& ph2, int& tt2, int& ks2) -> bool {
    ph2 = ph;
    tt2 = t;
    ks2 = ks + d;
    const int sp = ph == 0 ? s1p : s2p;
    if (ks2 >= sp) {
      ks2 -= sp;
      if (++tt2 == (ph == 0 ? t1 : t2)) {
        tt2 = 0;
        if (++ph2 == 2) {
          ph2 = 0;
          return true;
        }
      }
    }
    return false;
  };

  // weight chunks of stage ks of tile t of GEMM ph (MXFP4: of the double
  // stage that starts at the even stage ks)
  auto load_w = [&](const FfnUnit& u, int ph, int t, int ks, bool live, WS& ws) {
    const int N = ph == 0 ? N1 : L;
    const uint32_t rb = ph == 0 ? rb1 : rb2;
    const bool lv = live && u.valid && ks < (ph == 0 ? s1 : s2);
    const uint32_t ue = u.valid ? static_cast<uint32_t>(u.e) : 0u;
    if constexpr (FP4) {
      // elements 32 fq .. 32 fq + 31 of the double stage: 16 bytes, scale
      // block 4 j + fq of the row
      const uint32_t j = static_cast<uint32_t>(ks) >> 1;
      const uint32_t wbase = ue * (ph == 0 ? wm1 : wm2) + 64u * j + 16u * fq;
      const bool in_k = 128u * j + 32u * fq < static_cast<uint32_t>(ph == 0 ? L : M);
#pragma unroll
      for (int nb = 0; nb < kNWB; ++nb) {
        const int n = t * kTileN + nl + nb * 16;
        const bool in = lv && in_k && n < N;
        const uint32_t vo = in ? wbase + static_cast<uint32_t>(n) * rb : kOutOfRange;
        ws.b[nb] = buffer_load_chunk(ph == 0 ? w1r : w2r, vo, 0u);
      }
    } else {
      const uint32_t so = ue * (ph == 0 ? wm1 : wm2) + static_cast<uint32_t>(ks) * (kKE * 2) + 16u * fq;
#pragma unroll
      for (int nb = 0; nb < kNWB; ++nb) {
        const int n = t * kTileN + nl + nb * 16;
        const uint32_t vo = (lv && n < N) ? static_cast<uint32_t>(n) * rb + so : kOutOfRange;
        if (ph == 0) {
#pragma unroll
          for (int j = 0; j < kNLD; ++j) ws.b[nb][j] = buffer_load_chunk(w1r, vo + 64u * j, 0u);
        } else {
#pragma unroll
          for (int j = 0; j < kNLD; ++j) ws.b[nb][j] = buffer_load_chunk(w2r, vo + 64u * j, 0u);
        }
      }
    }
  };
  // MXFP4 block scales of a group of four double stages (eight stages, the
  // first one ks) of tile t of GEMM ph.  Lane fq of row n needs byte
  // 4 i + fq of the group's 16 (double stage 4 g + i) and keeps it in byte
  // fq of dword i.  Where the group's bytes are 16-byte aligned (scale rows
  // a multiple of 16 bytes, aligned array) every lane loads all 16 with one
  // request per row: a byte load per lane and double stage cost as many
  // requests as the weights themselves.  Otherwise four byte loads per lane.
  // Bytes past the row's K / 32 blocks belong to weights that read as zero
  // and are masked where the scales are decoded.
  const bool sgv1 = sb1 % 16u == 0 && (reinterpret_cast<uintptr_t>(p.W1_mx) & 15u) == 0;
  const bool sgv2 = sb2 % 16u == 0 && (reinterpret_cast<uintptr_t>(p.W2_mx) & 15u) == 0;
  auto load_sg = [&](const FfnUnit& u, int ph, int t, int ks, bool live, u32x4* dst) {
    const int N = ph == 0 ? N1 : L;
    const uint32_t sb = ph == 0 ? sb1 : sb2;
    const bool lv = live && u.valid && ks < (ph == 0 ? s1 : s2);
    const uint32_t ue = u.valid ? static_cast<uint32_t>(u.e) : 0u;
    const uint32_t base = ue * (ph == 0 ? sm1 : sm2) + 16u * (static_cast<uint32_t>(ks) >> 3);
    const BufRsrc r = ph == 0 ? s1r : s2r;
    if (ph == 0 ? sgv1 : sgv2) {
#pragma unroll
      for (int nb = 0; nb < kNWB; ++nb) {
        const int n = t * kTileN + nl + nb * 16;
        const uint32_t vo = (lv && n < N) ? base + static_cast<uint32_t>(n) * sb : kOutOfRange;
        dst[nb] = buffer_load_chunk(r, vo, 0u);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < kNWB; ++nb) {
        const int n = t * kTileN + nl + nb * 16;
        const uint32_t vo = (lv && n < N) ? base + static_cast<uint32_t>(n) * sb + fq : kOutOfRange;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[nb][i] = buffer_load_byte(r, vo + 4u * i) << (8u * fq);
      }
    }
  };
  // this thread's token chunk of FC1 stage ks (FC2 stages stage nothing)
  auto load_a = [&](const FfnUnit& u, int ph, int ks) -> u32x4 {
    uint32_t so, el;  // byte offset of the stage in a token row, element of the chunk
    if constexpr (FP4) {
      so = 256u * (static_cast<uint32_t>(ks) >> 1) + 32u * (ks & 1);
      el = so / 2u + 8u * a_chunk;
    } else {
      so = static_cast<uint32_t>(ks) * (kKE * 2);
      el = so / 2u + 8u * ac;
    }
    const bool in_k = ph == 0 && el < static_cast<uint32_t>(L);
    return buffer_load_chunk(a_rsrc, in_k ? u.a_off + so : kOutOfRange, 0u);
  };
  auto store_a = [&](int buf, const u32x4& v) {
    if (a_thread) As[buf][ar * 8 + (ac ^ ((ar >> 1) & 7))] = v;
  };

  f32x4_t acc[kMB][kNWB];
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < kNWB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one stage: weights first (rows n), token rows second, so that a lane
  // ends with D[n = 4 fq + v][row = fr] of each 16 x 16 block
  // nmb: 16-row token blocks of the pass that hold rows (the MFMAs of the
  // empty ones are skipped; their accumulators stay zero)
  u32x4 sgc[kNWB], sgn[kNWB];  // MXFP4 scales: current and next group
  float dsc[kNWB];              // MXFP4: scales of the current double stage
  auto compute = [&](int ph, int ks, int u, int buf, WS& ws, int nmb) {
    // token (FC1) or H (FC2) fragments: chunk of the stage for k-step s is
    // reduction elements 32 s + 8 fq .. (bf16 weights), or (MXFP4) elements
    // 32 fq + 16 (ks % 2) + 8 s .. of the double stage: staged chunk
    // 2 fq + s, H chunk hc of the row
    auto frag = [&](int s, int mb) -> u32x4 {
      const int c = FP4 ? 2 * fq + s : 4 * s + fq;
      const int hc = FP4 ? 16 * (ks >> 1) + 4 * fq + 2 * (ks & 1) + s : ks * 8 + c;
      const int r = mb * 16 + fr;
      return ph == 0 ? As[buf][r * 8 + (c ^ ((r >> 1) & 7))] : Hs[r * hcpr + (hc ^ (r & 7))];
    };
    // The fragments are read ahead of the MFMAs that use them, behind a
    // scheduling fence: left alone, the scheduler sinks each read to its
    // first use and waits for it there, six LDS round trips in a row per
    // stage.  MXFP4 reads the whole stage at once; bf16 (whose weight
    // registers leave less room) one k-step at a time.
    constexpr int kAhead = FP4 ? kNS : 1;
    u32x4 af[kNS][kMB];
#pragma unroll
    for (int s = 0; s < kAhead; ++s)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) af[s][mb] = frag(s, mb);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FP4) {
      // the first stage of a double stage decodes its scale bytes (u is the
      // stage within the group, ks = u modulo 8); blocks past K scale by 0
      if ((u & 1) == 0) {
        const bool in_k = 128 * (ks >> 1) + 32 * fq < (ph == 0 ? L : M);
#pragma unroll
        for (int nb = 0; nb < kNWB; ++nb) {
          const uint32_t e = __builtin_amdgcn_ubfe(sgc[nb][(u >> 1) & 3], 8u * fq, 8u);
          dsc[nb] = in_k ? e8m0_to_f32(e) : 0.f;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      if (s >= kAhead) {
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) af[s][mb] = frag(s, mb);
        __builtin_amdgcn_sched_barrier(0);
      }
      u32x4 bfr[kNWB];
#pragma unroll
      for (int nb = 0; nb < kNWB; ++nb) {
        if constexpr (FP4) bfr[nb] = fp4x8_to_bf16x8(ws.b[nb][2 * (ks & 1) + s], dsc[nb]);
        else bfr[nb] = ws.b[nb][s];
      }
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        if (mb > 0 && mb >= nmb) break;
#pragma unroll
        for (int nb = 0; nb < kNWB; ++nb) MmaBf16::mma(acc[mb][nb], bfr[nb], af[s][mb]);
      }
    }
  };

  // ---- first unit
  FfnUnit cur, nxt;
  set_expert(cur, blockIdx.x);
  if (!cur.valid) return;
  WS bw[NSLOT];
  u32x4 ra[2];
  // its first weight stages depend on the expert alone
  constexpr int kStep = FP4 ? 2 : 1;
#pragma unroll
  for (int i = 0; i < KWD; i += kStep) load_w(cur, 0, 0, i, true, bw[i / kStep]);
  if constexpr (FP4) load_sg(cur, 0, 0, 0, true, sgn);
  issue_bounds(cur);
  take_bounds(cur);
  if (cur.cnt <= 0) {  // no rows: the first expert with rows takes the prefetch
    find_rows(cur);
    if (!cur.valid) return;
#pragma unroll
    for (int i = 0; i < KWD; i += kStep) load_w(cur, 0, 0, i, true, bw[i / kStep]);
    if constexpr (FP4) load_sg(cur, 0, 0, 0, true, sgn);
  }
  issue_rows(cur);
  take_rows(cur);
  ra[0] = load_a(cur, 0, 0);
  ra[1] = load_a(cur, 0, 1);
  // H columns m .. mh-1 meet W2's columns past m as zeros; the FC1 epilogue
  // never writes them
  if (mh > M) {
    const int per = (mh - M) / 4;
    for (int q = tid; q < kRows * per; q += kThreads) {
      const int r = q / per, n0 = M + 4 * (q % per);
      *(reinterpret_cast<uint2*>(&Hs[r * hcpr + ((n0 >> 3) ^ (r & 7))]) + ((n0 >> 2) & 1)) =
          uint2{0u, 0u};
    }
  }
  store_a(0, ra[0]);
  lds_barrier();
  nxt.assign(cur);

  for (;;) {
    int q = 0;  // stage of this unit (a unit has at least 4 stages)
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int nt = ph == 0 ? t1 : t2;
      const int sp = ph == 0 ? s1p : s2p;
      for (int t = 0; t < nt; ++t) {
        for (int ks0 = 0; ks0 < sp; ks0 += KP) {
#pragma unroll
          for (int u = 0; u < KP; ++u) {
            const int ks = ks0 + u;
            // the next unit, read during the first three stages of this one
            // (its loads start in this unit's last kWD stages)
            if (q < 3) {
              if (q == 0) {
                if (cur.p0 + kRows < cur.cnt) {  // another pass over the same expert
                  nxt.assign(cur);
                  nxt.p0 = cur.p0 + kRows;
                  nxt.rows = min(kRows, cur.cnt - nxt.p0);
                } else {
                  set_expert(nxt, cur.e + gridDim.x);
                  issue_bounds(nxt);
                }
              } else if (q == 1) {
                if (nxt.p0 == 0) {
                  take_bounds(nxt);
                  find_rows(nxt);
                }
                issue_rows(nxt);
              } else {
                take_rows(nxt);
              }
            }
            ++q;
            // MXFP4: a group of eight stages starts; its scales were loaded
            // eight stages ago, the next group's are loaded now
            if constexpr (FP4) {
              static_assert(KP == 8, "a scale group is one unrolled iteration");
              if (u == 0) {
#pragma unroll
                for (int nb = 0; nb < kNWB; ++nb) sgc[nb] = sgn[nb];
                int ph2, tt2, ks2;
                const bool nx = advance(ph, t, ks, KP, ph2, tt2, ks2);
                if (nx) load_sg(nxt, ph2, tt2, ks2, nxt.rows > 0, sgn);
                else load_sg(cur, ph2, tt2, ks2, cur.rows > 0, sgn);
              }
            }
            // weights of the stage KWD ahead (MXFP4: at even stages, the
            // double stage KWD ahead), token rows of the stage 2 ahead
            if (u % kStep == 0) {
              int ph2, tt2, ks2;
              const bool nx = advance(ph, t, ks, KWD, ph2, tt2, ks2);
              WS& dst = bw[(u + KWD) / kStep % NSLOT];
              if (nx) load_w(nxt, ph2, tt2, ks2, nxt.rows > 0, dst);
              else load_w(cur, ph2, tt2, ks2, cur.rows > 0, dst);
            }
            {
              int ph2, tt2, ks2;
              const bool nx = advance(ph, t, ks, 2, ph2, tt2, ks2);
              ra[u % 2] = nx ? load_a(nxt, ph2, ks2) : load_a(cur, ph2, ks2);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks < (ph == 0 ? s1 : s2))
              compute(ph, ks, u, u % 2, bw[u / kStep % NSLOT], (cur.rows + 15) >> 4);
            store_a((u + 1) % 2, ra[(u + 1) % 2]);
            // FC1 stages read the staged token rows; FC2 stages read only H,
            // so the waves run through FC2 unsynchronised until its last
            // stage, after which the next unit's first token stage is read
            if (ph == 0 || (t == nt - 1 && ks == sp - 1)) lds_barrier();
          }
        }
        // tile epilogue: lane holds D[n = 4 fq + v][row = fr] of block (mb, nb)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          const int r = mb * 16 + fr;
#pragma unroll
          for (int nb = 0; nb < kNWB; ++nb) {
            const int n0 = t * kTileN + wave * (kNWB * 16) + nb * 16 + 4 * fq;
            const f32x4_t a = acc[mb][nb];
            if (ph == 0) {
              if (GLU) {
                // columns (n0, n0 + 1), (n0 + 2, n0 + 3) are (up, gate) pairs:
                // H columns n0 / 2 and n0 / 2 + 1, one 4-byte piece
                const int c = n0 >> 1;
                if (n0 < N1)
                  *(reinterpret_cast<uint32_t*>(&Hs[r * hcpr + ((c >> 3) ^ (r & 7))]) + ((c >> 1) & 3)) =
                      pack_bf16x2(swiglu(a[0], a[1]), swiglu(a[2], a[3]));
              } else if (n0 < M) {
                const uint2 h{pack_bf16x2(apply_act<kActSqRelu>(a[0]), apply_act<kActSqRelu>(a[1])),
                              pack_bf16x2(apply_act<kActSqRelu>(a[2]), apply_act<kActSqRelu>(a[3]))};
                *(reinterpret_cast<uint2*>(&Hs[r * hcpr + ((n0 >> 3) ^ (r & 7))]) + ((n0 >> 2) & 1)) = h;
              }
            } else if (r < cur.rows && n0 < L) {
              const uint2 y{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
              *reinterpret_cast<uint2*>(Y + ((int64_t)cur.gs + cur.p0 + r) * p.ldy + n0) = y;
            }
            acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
        if (ph == 0 && t == nt - 1) lds_barrier();  // H complete before FC2 reads it
      }
    }
    if (!nxt.valid) break;
    cur.assign(nxt);
  }
}

}  // namespace

bool ffn_stream_fits(int G, int l, int m, bool glu, bool fp4) {
  if (G < 1 || l <= 0 || m <= 0 || m > kMaxM || l % 16 || m % 16) return false;
  if (fp4 && (l % 32 || m % 32)) return false;  // whole MX scale blocks per row
  // each weight array (all experts) below 2 GiB: 32-bit offsets from one
  // buffer resource per array
  const uint64_t n1 = glu ? 2ull * m : uint64_t(m);
  const uint64_t rb1 = fp4 ? uint64_t(l) / 2 : 2ull * l, rb2 = fp4 ? uint64_t(m) / 2 : 2ull * m;
  return uint64_t(G) * n1 * rb1 < (1ull << 31) && uint64_t(G) * uint64_t(l) * rb2 < (1ull << 31);
}

int ffn_stream_rows() { return kRows; }

hipError_t launch_ffn_stream(const FfnArgs& a, hipStream_t s) {
  if (a.act != kActSqRelu && a.act != kActSwiGlu) return hipErrorInvalidValue;
  const bool glu = a.act == kActSwiGlu;
  const bool fp4 = a.W1_mx != nullptr;
  if (!ffn_stream_fits(a.G, a.l, a.m, glu, fp4) || !a.g_off || !a.a_rows || a.ldy % 4 ||
      a.lda < a.l || (fp4 && !a.W2_mx))
    return hipErrorInvalidValue;
  // 32-bit buffer offsets: token rows stay below 2 GiB
  if ((uint64_t)a.a_nrows * a.lda * 2u >= (1ull << 31)) return hipErrorInvalidValue;
  const int grid = std::min(a.G, device_compute_units());
  if (fp4) {
    if (glu) ffn_stream_kernel<true, true><<<dim3(grid), dim3(kThreads), 0, s>>>(a);
    else ffn_stream_kernel<false, true><<<dim3(grid), dim3(kThreads), 0, s>>>(a);
  } else {
    if (glu) ffn_stream_kernel<true, false><<<dim3(grid), dim3(kThreads), 0, s>>>(a);
    else ffn_stream_kernel<false, false><<<dim3(grid), dim3(kThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace lmoe
