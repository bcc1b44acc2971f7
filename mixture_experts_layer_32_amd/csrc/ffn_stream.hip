// Fused latent expert FFN for the decode regime, for gfx950:
//
//   H = sqrelu(A_g W1_g^T)   rows of expert g  x  m   (kept in LDS, bf16)
//   Y = H W2_g^T             rows of expert g  x  l   (written to HBM, bf16)
//
// (the expert FFN of the LatentMoE paper, Eq. (2): both expert GEMMs run in
// the latent width l, with the squared-ReLU activation of Table 2).  With
// SwiGLU experts W1 holds 2m rows, up-projection and gate rows interleaved,
// and H[i] = up_i * SiLU(gate_i): FC1 streams twice the rows.  With MXFP4
// weights (E2M1 pairs, an E8M0 scale per 32 elements) a lane takes 16
// consecutive elements of a row per stage (one 8-byte load and its block's
// scale byte) and widens them to two bf16 MFMA operands; the token and H
// fragments then take the matching reduction indices.
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
//    64 contiguous bytes of a row, WD stages ahead of the one multiplied.
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

#ifndef LMOE_FFN_NWB
#define LMOE_FFN_NWB 4
#endif
#ifndef LMOE_FFN_WD
#define LMOE_FFN_WD 3
#endif
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMB = 3;                         // 16-row blocks of token rows per pass
constexpr int kRows = 16 * kMB;                // token rows per pass
constexpr int kNWB = LMOE_FFN_NWB;             // 16-row weight blocks per wave
constexpr int kTileN = kWaves * kNWB * 16;     // output columns per tile
constexpr int kKE = 64;                        // reduction elements per stage
constexpr int kNS = kKE / 32;                  // MFMA k-steps per stage
constexpr int kNLD = kNS;                      // 16-byte weight loads per n-block per stage
constexpr int kWD = LMOE_FFN_WD;               // weight stages in flight ahead
// registers rotate: weights modulo kWD + 1 stages, staged token rows modulo 2
constexpr int kP = (kWD + 1) % 2 == 0 ? kWD + 1 : 2 * (kWD + 1);
constexpr int kMaxM = 1536;                    // hidden width that fits in LDS
constexpr int kAChunks = kRows * (kKE / 8);    // staged token chunks per stage (384)

struct FfnUnit {
  int e;             // expert (group)
  int valid;         // 0: past the last expert
  int gs, cnt;       // first grouped row of the expert and its row count
  int p0, rows;      // this pass's first row (within the expert) and its rows
  BufRsrc w1, w2;    // the expert's weight matrices
  BufRsrc s1, s2;    // MXFP4: their block scales
  uint32_t a_off;       // this thread's staged token chunk, or out of range

  __device__ __forceinline__ void assign(const FfnUnit& o) {
    e = o.e;
    valid = o.valid;
    gs = o.gs;
    cnt = o.cnt;
    p0 = o.p0;
    rows = o.rows;
    w1 = o.w1;
    w2 = o.w2;
    s1 = o.s1;
    s2 = o.s2;
    a_off = o.a_off;
  }
};

// Weight registers of one stage: bf16 rows (kNLD 16-byte chunks per n-block),
// or MXFP4 rows (one 8-byte piece and its scale byte per n-block)
struct WStageBf16 {
  u32x4 b[kNWB][kNLD];
};
struct WStageFp4 {
  u32x2 b[kNWB];
  uint32_t s[kNWB];
};

template <bool GLU, bool FP4>
__global__ __launch_bounds__(kThreads, 1) void ffn_stream_kernel(FfnArgs p) {
  using WS = std::conditional_t<FP4, WStageFp4, WStageBf16>;
  __shared__ u32x4 Hs[kRows * kMaxM / 8];  // H, 16-byte chunk c of row r at c ^ (r & 7)
  __shared__ u32x4 As[2][kAChunks];        // FC1 token stages, chunk c of row r at c ^ ((r >> 1) & 7)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fq = lane >> 4;
  const int L = p.l, M = p.m;
  const int N1 = GLU ? 2 * M : M;            // FC1 weight rows (H columns x 2 with SwiGLU)
  const int mh = (M + kKE - 1) / kKE * kKE;  // H row length: m rounded up to a stage
  const int hcpr = mh / 8;                   // 16-byte chunks per H row
  const int s1 = (L + kKE - 1) / kKE;        // FC1 stages (reduction over l)
  const int s2 = mh / kKE;                   // FC2 stages (reduction over m)
  const int s1p = (s1 + kP - 1) / kP * kP;
  const int s2p = (s2 + kP - 1) / kP * kP;
  const int t1 = (N1 + kTileN - 1) / kTileN; // FC1 tiles (of W1 rows)
  const int t2 = (L + kTileN - 1) / kTileN;  // FC2 tiles (Y columns)
  const uint32_t rb1 = FP4 ? static_cast<uint32_t>(L) / 2u : static_cast<uint32_t>(L) * 2u;  // W1 row bytes
  const uint32_t rb2 = FP4 ? static_cast<uint32_t>(M) / 2u : static_cast<uint32_t>(M) * 2u;  // W2 row bytes
  const uint32_t sb1 = static_cast<uint32_t>(L) / 32u;  // MXFP4: scale bytes per W1 row
  const uint32_t sb2 = static_cast<uint32_t>(M) / 32u;  // and per W2 row
  const uint32_t a_row_bytes = static_cast<uint32_t>(p.lda) * 2u;
  const BufRsrc a_rsrc = make_rsrc(p.A, (uint64_t)p.a_nrows * p.lda * 2u);
  const BufRsrc goff_rsrc = make_rsrc(p.g_off, (uint64_t)(p.G + 1) * sizeof(int32_t));
  const uint8_t* const w1g = static_cast<const uint8_t*>(p.W1);
  const uint8_t* const w2g = static_cast<const uint8_t*>(p.W2);
  uint16_t* const Y = static_cast<uint16_t*>(p.Y);
  const int nl = wave * (kNWB * 16) + fr;    // weight row of n-block 0 within a tile
  const int ar = tid >> 3, ac = tid & 7;     // staged token chunk of this thread
  const bool a_thread = tid < kAChunks;

  // ---- unit bookkeeping
  auto set_expert = [&](FfnUnit& u, int e) {
    u.e = e;
    u.valid = e < p.G;
    const int64_t ee = u.valid ? e : 0;
    u.w1 = make_rsrc(w1g + ee * N1 * rb1, (uint64_t)N1 * rb1);
    u.w2 = make_rsrc(w2g + ee * L * rb2, (uint64_t)L * rb2);
    if constexpr (FP4) {
      u.s1 = make_rsrc(p.W1_mx + ee * N1 * sb1, (uint64_t)N1 * sb1);
      u.s2 = make_rsrc(p.W2_mx + ee * L * sb2, (uint64_t)L * sb2);
    }
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
  auto take_rows = [&](FfnUnit& u) {
    u.a_off = (a_thread && ar < u.rows) ? static_cast<uint32_t>(tok) * a_row_bytes + 16u * ac
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

  // weight chunks of stage ks of tile t of GEMM ph
  auto load_w = [&](const FfnUnit& u, int ph, int t, int ks, bool live, WS& ws) {
    const int N = ph == 0 ? N1 : L;
    const uint32_t rb = ph == 0 ? rb1 : rb2;
    const bool lv = live && ks < (ph == 0 ? s1 : s2);
    if constexpr (FP4) {
      // elements 16 fq .. 16 fq + 15 of the stage: 8 bytes, one scale block
      const uint32_t sb = ph == 0 ? sb1 : sb2;
      const uint32_t so = static_cast<uint32_t>(ks) * (kKE / 2) + 8u * fq;
      const uint32_t ss = static_cast<uint32_t>(ks) * (kKE / 32) + (fq >> 1);
#pragma unroll
      for (int nb = 0; nb < kNWB; ++nb) {
        const int n = t * kTileN + nl + nb * 16;
        const bool in = lv && n < N;
        const uint32_t vo = in ? static_cast<uint32_t>(n) * rb + so : kOutOfRange;
        const uint32_t vs = in ? static_cast<uint32_t>(n) * sb + ss : kOutOfRange;
        ws.b[nb] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(ph == 0 ? u.w1 : u.w2,
                                                        static_cast<int>(vo), 0, 0));
        ws.s[nb] = buffer_load_byte(ph == 0 ? u.s1 : u.s2, vs);
      }
    } else {
      const uint32_t so = static_cast<uint32_t>(ks) * (kKE * 2) + 16u * fq;
#pragma unroll
      for (int nb = 0; nb < kNWB; ++nb) {
        const int n = t * kTileN + nl + nb * 16;
        const uint32_t vo = (lv && n < N) ? static_cast<uint32_t>(n) * rb + so : kOutOfRange;
        if (ph == 0) {
#pragma unroll
          for (int j = 0; j < kNLD; ++j) ws.b[nb][j] = buffer_load_chunk(u.w1, vo + 64u * j, 0u);
        } else {
#pragma unroll
          for (int j = 0; j < kNLD; ++j) ws.b[nb][j] = buffer_load_chunk(u.w2, vo + 64u * j, 0u);
        }
      }
    }
  };
  // this thread's token chunk of FC1 stage ks (FC2 stages stage nothing)
  auto load_a = [&](const FfnUnit& u, int ph, int ks) -> u32x4 {
    const bool in_k = ph == 0 && ks * kKE + ac * 8 < L;
    return buffer_load_chunk(
        a_rsrc, in_k ? u.a_off + static_cast<uint32_t>(ks) * (kKE * 2) : kOutOfRange, 0u);
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
  auto compute = [&](int ph, int ks, int buf, const WS& ws) {
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      // chunk of the stage: reduction elements 32 s + 8 fq .. (bf16 weights),
      // 16 fq + 8 s .. (MXFP4: a lane's 16 consecutive elements)
      const int c = FP4 ? 2 * fq + s : 4 * s + fq;
      u32x4 bfr[kNWB];
#pragma unroll
      for (int nb = 0; nb < kNWB; ++nb) {
        if constexpr (FP4) bfr[nb] = fp4x8_to_bf16x8(ws.b[nb][s], e8m0_to_f32(ws.s[nb]));
        else bfr[nb] = ws.b[nb][s];
      }
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const int r = mb * 16 + fr;
        const u32x4 a = ph == 0 ? As[buf][r * 8 + (c ^ ((r >> 1) & 7))]
                                : Hs[r * hcpr + ((ks * 8 + c) ^ (r & 7))];
#pragma unroll
        for (int nb = 0; nb < kNWB; ++nb) MmaBf16::mma(acc[mb][nb], bfr[nb], a);
      }
    }
  };

  // ---- first unit
  FfnUnit cur, nxt;
  set_expert(cur, blockIdx.x);
  if (!cur.valid) return;
  WS bw[kWD + 1];
  u32x4 ra[2];
  // its first weight stages depend on the expert alone
#pragma unroll
  for (int i = 0; i < kWD; ++i) load_w(cur, 0, 0, i, true, bw[i]);
  issue_bounds(cur);
  take_bounds(cur);
  if (cur.cnt <= 0) {  // no rows: the first expert with rows takes the prefetch
    find_rows(cur);
    if (!cur.valid) return;
#pragma unroll
    for (int i = 0; i < kWD; ++i) load_w(cur, 0, 0, i, true, bw[i]);
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
    for (int ph = 0; ph < 2; ++ph) {
      const int nt = ph == 0 ? t1 : t2;
      const int sp = ph == 0 ? s1p : s2p;
      for (int t = 0; t < nt; ++t) {
        for (int ks0 = 0; ks0 < sp; ks0 += kP) {
#pragma unroll
          for (int u = 0; u < kP; ++u) {
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
            // weights of the stage kWD ahead, token rows of the stage 2 ahead
            {
              int ph2, tt2, ks2;
              const bool nx = advance(ph, t, ks, kWD, ph2, tt2, ks2);
              if (nx) load_w(nxt, ph2, tt2, ks2, nxt.rows > 0, bw[(u + kWD) % (kWD + 1)]);
              else load_w(cur, ph2, tt2, ks2, cur.rows > 0, bw[(u + kWD) % (kWD + 1)]);
            }
            {
              int ph2, tt2, ks2;
              const bool nx = advance(ph, t, ks, 2, ph2, tt2, ks2);
              ra[u % 2] = nx ? load_a(nxt, ph2, ks2) : load_a(cur, ph2, ks2);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks < (ph == 0 ? s1 : s2)) compute(ph, ks, u % 2, bw[u % (kWD + 1)]);
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

bool ffn_stream_fits(int l, int m) {
  return l > 0 && m > 0 && m <= kMaxM && l % 16 == 0 && m % 16 == 0;
}

int ffn_stream_rows() { return kRows; }

hipError_t launch_ffn_stream(const FfnArgs& a, hipStream_t s) {
  if (!ffn_stream_fits(a.l, a.m) || a.G < 1 || !a.g_off || !a.a_rows || a.ldy % 4 ||
      a.lda < a.l || (a.act != kActSqRelu && a.act != kActSwiGlu))
    return hipErrorInvalidValue;
  const bool glu = a.act == kActSwiGlu;
  const bool fp4 = a.W1_mx != nullptr;
  // MXFP4: both scale arrays, whole scale blocks per row
  if (fp4 && (!a.W2_mx || a.l % 32 || a.m % 32)) return hipErrorInvalidValue;
  // 32-bit buffer offsets: token rows and one expert matrix stay below 2 GiB
  if ((uint64_t)a.a_nrows * a.lda * 2u >= (1ull << 31) ||
      (uint64_t)(glu ? 2 : 1) * a.m * a.l * 2u >= (1ull << 31))
    return hipErrorInvalidValue;
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
