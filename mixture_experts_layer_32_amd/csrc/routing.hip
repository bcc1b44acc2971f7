// Routing and combine kernels of the LatentMoE layer, for gfx950.
//
// LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in Mixture of
// Experts, §3: routing weights from the router logits, the top-K expert set
// T_{K,N'} of each token, dispatch of the latent token copies to their
// experts and the gate-weighted aggregation sum_{i in T} p'_i E_i(u).
//
//  topk_gate     one wave per token: the K-th largest logit by a bitwise
//                search over order-preserving keys (ballot counts), the set
//                (ties at the K-th place to the lower ids), each member's
//                rank under (logit desc, expert id asc), then the gate rule.
//  route_masks   per block of 64 tokens, one 64-bit mask per expert of the
//                tokens that chose it (LDS 64-bit atomic OR; integer, exact).
//  route_scan    per (block, expert) the copies of that expert in earlier
//                blocks and the expert counts (popcounts, a column scan over
//                the blocks spread over workgroups of 64 experts), then one
//                workgroup: exclusive prefix sum over experts (offsets).
//  route_assign  one thread per copy (t, j): its row is the expert's offset
//                plus the copies of the expert in earlier blocks plus the
//                earlier tokens of its own block that chose the expert, so
//                rows of an expert follow increasing token index.
//  route_small   the three steps above in one launch when all masks fit in
//                LDS (decode-sized batches).
//  combine       v[t] = sum_j gate[t][j] * Y[slot_of[t][j]] in fp32, fixed
//                j order (deterministic), plus an optional fp32 residual (the
//                shared experts' sum when v is the layer output), rounded
//                once to the output dtype.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

constexpr int kTopkMaxPerLane = 32;     // N <= 2048
constexpr int kSmallRouteMasks = 4096;  // route_small: routing blocks x experts
constexpr int kSmallRouteCopies = 16384; // route_small: token copies T x K

// fp32 -> uint32 whose unsigned order is the float order (+0 == -0); zero
// is never the key of a number, so it marks "no value".
__device__ __forceinline__ uint32_t order_key(float z) {
  if (z == 0.f) z = 0.f;
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Blocks past tok_blocks finish the down-projection instead: one 4-column
// piece of u per thread, its split-K partials added in split order (the
// order of the GEMM's own reduction kernel).  SPL > 1: the logits arrive in
// at most SPL partial sets, all loaded before they are added in order.
template <int NPL, int SPL>
__global__ __launch_bounds__(256) void topk_gate_kernel(TopkArgs a, int tok_blocks) {
  const int T = a.T, N = a.N, K = a.K;
  if (static_cast<int>(blockIdx.x) >= tok_blocks) {
    const int l4 = a.l / 4;
    const int64_t q = (int64_t)(blockIdx.x - tok_blocks) * 256 + threadIdx.x;
    if (q >= (int64_t)T * l4) return;
    const int r = static_cast<int>(q / l4), c = static_cast<int>(q % l4) * 4;
    const float* pp = a.u_part + (int64_t)r * a.u_ld + c;
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(pp);
    for (int z = 1; z < a.usplits; ++z) v += *reinterpret_cast<const f32x4_t*>(pp + z * a.u_sstride);
    if (a.u_bf16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.u) + (int64_t)r * a.l + c) =
          uint2{uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16),
                uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16)};
    } else {
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.u) + (int64_t)r * a.l + c) = v;
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves leave together

  // value i of this lane is expert 64 i + lane; loads are unconditional
  // (clamped index) so they are all in flight together.  Split-K partials
  // of the logits are added in split order.
  const float* zr = a.logits + (int64_t)t * a.logits_ld;
  const int64_t tn = a.logits_sstride;
  float zs[NPL];
  if constexpr (SPL > 1) {
    float pz[SPL][NPL];
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp)
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = i * 64 + lane;
        const int ec = e < N ? e : N - 1;
        pz[sp][i] = zr[(sp < a.lsplits ? sp : 0) * tn + ec];
      }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      float v = pz[0][i];
#pragma unroll
      for (int sp = 1; sp < SPL; ++sp)
        if (sp < a.lsplits) v += pz[sp][i];
      zs[i] = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = i * 64 + lane;
      const int ec = e < N ? e : N - 1;
      float v = zr[ec];
      for (int sp = 1; sp < a.lsplits; ++sp) v += zr[sp * tn + ec];
      zs[i] = v;
    }
  }
  float z[NPL];
  uint32_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = i * 64 + lane;
    const int ec = e < N ? e : N - 1;
    float v = zs[i];
    if (a.logits_out && e < N) a.logits_out[(int64_t)t * N + e] = v;
    v += a.bias ? a.bias[ec] : 0.f;
    z[i] = e < N ? v : -INFINITY;
    key[i] = e < N ? order_key(v) : 0u;
  }
  const int gating = a.gating;

  // ---- the selected set: tau = the K-th largest key, the largest v with
  // #{keys >= v} >= K, found bit by bit from the top (counts are ballot
  // popcounts); a candidate with exactly K keys at or above it ends the
  // search, those keys being the set.  Otherwise the set is every key above
  // tau and, of the keys equal to tau, the lowest ids (id = 64 i + lane:
  // value index first, then lane).
  auto count_ge = [&](uint32_t v) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) c += __popcll(__ballot(key[i] >= v));
    return c;
  };
  uint32_t tau = 0;
  bool exact = false;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    const int c = count_ge(cand);
    if (c >= K) {
      tau = cand;
      if (c == K) { exact = true; break; }
    }
  }
  bool sel[NPL];
  if (exact) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) sel[i] = key[i] >= tau;
  } else {
    int r = K - (tau == 0xffffffffu ? 0 : count_ge(tau + 1u));  // ties still to take
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const bool eq = key[i] == tau;
      const uint64_t m = __ballot(eq);
      const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
          static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
      sel[i] = key[i] > tau || (eq && below < r);
      r -= __popcll(m);
    }
  }
  // ---- the K selected values to lanes 0..K-1 (in id order, through this
  // wave's LDS row; one wave's LDS operations complete in order)
  __shared__ uint32_t s_key[4][64];
  __shared__ int s_id[4][64];
  __shared__ float s_z[4][64];
  const int w = threadIdx.x >> 6;
  {
    int pos = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const uint64_t m = __ballot(sel[i]);
      if (sel[i]) {
        const int q = pos + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                static_cast<uint32_t>(m >> 32),
                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
        s_key[w][q] = key[i];
        s_id[w][q] = i * 64 + lane;
        s_z[w][q] = z[i];
      }
      pos += __popcll(m);
    }
  }
  const bool mine = lane < K;
  const uint32_t my_key = mine ? s_key[w][lane] : 0u;
  const int my_e = mine ? s_id[w][lane] : 0;
  const float my_z = mine ? s_z[w][lane] : 0.f;
  // rank under (key desc, id asc): the selected values that come before
  const uint64_t my_c = (static_cast<uint64_t>(my_key) << 32) | (0xffffffffu - static_cast<uint32_t>(my_e));
  int rank = 0;
  for (int q = 0; q < K; ++q) {
    const uint64_t c = (static_cast<uint64_t>(__builtin_amdgcn_readlane(my_key, q)) << 32) |
                       (0xffffffffu - static_cast<uint32_t>(__builtin_amdgcn_readlane(my_e, q)));
    rank += c > my_c ? 1 : 0;
  }

  // ---- gates (rule from the layer configuration); zmax is the first
  // selected logit
  const uint64_t first = __ballot(mine && rank == 0);
  const int l0 = __ffsll(static_cast<unsigned long long>(first)) - 1;
  const float zmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_z), l0));
  float g;
  if (gating == 2) {  // sigmoid, normalised over the selected set
    const float sgm = mine ? 1.f / (1.f + expf(-my_z)) : 0.f;
    g = sgm / wave_sum(sgm);
  } else {
    const float ex = mine ? expf(my_z - zmax) : 0.f;
    float tot;
    if (gating == 0) {  // softmax over all N logits, no renormalisation
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i * 64 + lane < N) part += expf(z[i] - zmax);
      tot = wave_sum(part);
    } else {            // softmax over the selected logits
      tot = wave_sum(ex);
    }
    g = ex / tot;
  }
  if (mine) {
    a.idx[(int64_t)t * K + rank] = my_e;
    a.gate[(int64_t)t * K + rank] = g;
  }
}

__global__ __launch_bounds__(256) void route_masks_kernel(const int32_t* __restrict__ idx, int T,
                                                          int N, int K,
                                                          uint64_t* __restrict__ masks) {
  extern __shared__ unsigned long long sm[];
  const int blk = blockIdx.x;
  for (int e = threadIdx.x; e < N; e += blockDim.x) sm[e] = 0ull;
  __syncthreads();
  const int t0 = blk * kRouteBlock;
  const int nt = min(kRouteBlock, T - t0);
  const int ncopy = nt * K;
  for (int q = threadIdx.x; q < ncopy; q += blockDim.x) {
    const int tl = q / K;
    const int e = idx[(int64_t)t0 * K + q];
    atomicOr(&sm[e], 1ull << tl);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) masks[(int64_t)blk * N + e] = sm[e];
}

// Exclusive scans over up to 2048 experts of the counts and of their tile
// counts, by a workgroup of 1024 threads: thread t holds the values of
// experts t and t + 1024 in cnt[0..1].  Results in s_cnt / s_til (exclusive
// prefix per expert) and the totals.
__device__ void expert_scan(const int (&cnt)[2], int N, int tile_m, int* s_cnt, int* s_til,
                            int (*s_wsum)[16], int& total_c, int& total_t) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + h * 1024;
    s_cnt[e] = e < N ? cnt[h] : 0;
    s_til[e] = e < N ? (cnt[h] + tile_m - 1) / tile_m : 0;
  }
  __syncthreads();
  // thread tid owns experts 2*tid and 2*tid+1 of the scan's linear order
  const int a0 = s_cnt[2 * tid], a1 = s_cnt[2 * tid + 1];
  const int t0 = s_til[2 * tid], t1 = s_til[2 * tid + 1];
  int pc = a0 + a1, pt = t0 + t1;
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {  // inclusive scan within the wave
    const int yc = __shfl_up(pc, o, kWave), yt = __shfl_up(pt, o, kWave);
    if (lane >= o) { pc += yc; pt += yt; }
  }
  if (lane == 63) { s_wsum[0][w] = pc; s_wsum[1][w] = pt; }
  __syncthreads();
  int wc = 0, wt = 0;
  for (int i = 0; i < w; ++i) { wc += s_wsum[0][i]; wt += s_wsum[1][i]; }
  const int exc = wc + pc - (a0 + a1), ext = wt + pt - (t0 + t1);
  s_cnt[2 * tid] = exc;  // every read of s_cnt/s_til happened before the last barrier
  s_cnt[2 * tid + 1] = exc + a0;
  s_til[2 * tid] = ext;
  s_til[2 * tid + 1] = ext + t0;
  total_c = 0;
  total_t = 0;
  for (int i = 0; i < 16; ++i) { total_c += s_wsum[0][i]; total_t += s_wsum[1][i]; }
  __syncthreads();
}

// Per expert, the copies in earlier routing blocks (base) and the total
// (counts): a column scan of the [nblk][N] mask popcounts.  Workgroup x
// takes experts 64 x .. 64 x + 63 (one per lane, so each load instruction
// reads 512 contiguous bytes) and its 16 waves split the blocks into 16
// ranges: a range's sum, the sums of the earlier ranges through LDS, then
// the range again (from L2) for the running values.
__global__ __launch_bounds__(1024) void route_colscan_kernel(const uint64_t* __restrict__ masks,
                                                             int nblk, int N,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ base) {
  __shared__ int s_part[16][64];
  const int lane = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int per = (nblk + 15) / 16;
  const int b0 = min(nblk, r * per), b1 = min(nblk, b0 + per);
  const int ec = e < N ? e : N - 1;  // loads stay in bounds; results of e >= N are dropped
  int sum = 0;
  for (int b = b0; b < b1; b += 8) {  // 8 independent loads in flight
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = b + u < b1 ? masks[(int64_t)(b + u) * N + ec] : 0ull;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += __popcll(v[u]);
  }
  s_part[r][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int i = 0; i < r; ++i) run += s_part[i][lane];
  if (e >= N) return;
  if (r == 15) counts[e] = run + sum;
  for (int b = b0; b < b1; b += 8) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = b + u < b1 ? masks[(int64_t)(b + u) * N + e] : 0ull;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (b + u < b1) base[(int64_t)(b + u) * N + e] = run;
      run += __popcll(v[u]);
    }
  }
}

// Exclusive prefix of the counts over the experts (offsets, tiles, the
// list of experts with copies): one workgroup of 1024 threads; N <= 2048.
__global__ __launch_bounds__(1024) void route_offsets_kernel(const int32_t* __restrict__ counts,
                                                             int N, int tile_m,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tiles,
                                                             int32_t* __restrict__ active) {
  __shared__ int s_cnt[2048];
  __shared__ int s_til[2048];
  __shared__ int s_wsum[2][16];
  const int tid = threadIdx.x;
  int cnt[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + h * 1024;
    cnt[h] = e < N ? counts[e] : 0;
  }
  int total_c, total_t;
  expert_scan(cnt, N, tile_m, s_cnt, s_til, s_wsum, total_c, total_t);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + h * 1024;
    if (e < N) {
      offsets[e] = s_cnt[e];
      if (tiles) tiles[e] = s_til[e];
      // one "tile" per expert with copies: s_til is its rank among them
      if (active && cnt[h] > 0) active[s_til[e]] = e;
    }
  }
  if (tid == 0) {
    offsets[N] = total_c;
    if (tiles) tiles[N] = total_t;
  }
}

__global__ __launch_bounds__(256) void route_assign_kernel(const int32_t* __restrict__ idx,
                                                           const uint64_t* __restrict__ masks,
                                                           const int32_t* __restrict__ base,
                                                           const int32_t* __restrict__ offsets,
                                                           int T, int N, int K,
                                                           int32_t* __restrict__ slot_of,
                                                           int32_t* __restrict__ token_of) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= (int64_t)T * K) return;
  const int t = static_cast<int>(q / K);
  const int e = idx[q];
  const int blk = t / kRouteBlock, tl = t % kRouteBlock;
  const uint64_t m = masks[(int64_t)blk * N + e];
  const int slot = offsets[e] + base[(int64_t)blk * N + e] + __popcll(m & ((1ull << tl) - 1ull));
  slot_of[q] = slot;
  token_of[slot] = t;
}

// masks + scan + assign for a decode-sized batch in one launch of
// ceil(T*K / 1024) workgroups of 1024 threads; requires
// ceil(T / 64) * N <= kSmallRouteMasks (the masks live in LDS) and
// T * K <= kSmallRouteCopies (16 copies per thread, held in registers).
// Every workgroup builds all masks and the expert scan itself (a few
// microseconds of LDS work on 64 KB of indices read from L2); workgroup b
// then assigns the copies q in [1024 b, 1024 b + 1024), so the scattered
// token_of stores are spread over several compute units.
__global__ __launch_bounds__(1024) void route_small_kernel(const int32_t* __restrict__ idx, int T,
                                                           int N, int K, int tile_m,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tiles,
                                                           int32_t* __restrict__ slot_of,
                                                           int32_t* __restrict__ token_of,
                                                           int32_t* __restrict__ active) {
  __shared__ unsigned long long sm[kSmallRouteMasks];
  __shared__ int s_cnt[2048];
  __shared__ int s_til[2048];
  __shared__ int s_wsum[2][16];
  __shared__ uint16_t s_pre[kSmallRouteMasks];
  const int tid = threadIdx.x;
  const int nblk = (T + kRouteBlock - 1) / kRouteBlock;
  const int nm = nblk * N;
  const int ncopy = T * K;
  // the copy this thread assigns, and every copy q = tid + 1024 i for the
  // masks, all requested in one batch
  const int my_q = blockIdx.x * 1024 + tid;
  const int my_e = idx[my_q < ncopy ? my_q : 0];
  int ids[kSmallRouteCopies / 1024];
#pragma unroll
  for (int i = 0; i < kSmallRouteCopies / 1024; ++i) {
    const int q = tid + 1024 * i;
    ids[i] = idx[q < ncopy ? q : 0];
  }
  for (int i = tid; i < nm; i += 1024) sm[i] = 0ull;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSmallRouteCopies / 1024; ++i) {
    const int q = tid + 1024 * i;
    if (q < ncopy) {
      const int t = q / K;
      atomicOr(&sm[(t / kRouteBlock) * N + ids[i]], 1ull << (t % kRouteBlock));
    }
  }
  __syncthreads();
  // per expert: its copies in earlier blocks (s_pre, < T <= 16384 so 16 bits
  // suffice) and its total count
  int cnt[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + h * 1024;
    if (e < N)
      for (int b = 0; b < nblk; ++b) {
        s_pre[b * N + e] = static_cast<uint16_t>(cnt[h]);
        cnt[h] += __popcll(sm[b * N + e]);
      }
  }
  int total_c, total_t;
  expert_scan(cnt, N, tile_m, s_cnt, s_til, s_wsum, total_c, total_t);
  if (blockIdx.x == 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + h * 1024;
      if (e < N) {
        counts[e] = cnt[h];
        offsets[e] = s_cnt[e];
        if (tiles) tiles[e] = s_til[e];
        if (active && cnt[h] > 0) active[s_til[e]] = e;
      }
    }
    if (tid == 0) {
      offsets[N] = total_c;
      if (tiles) tiles[N] = total_t;
    }
  }
  // s_cnt holds the exclusive offsets and is no longer written
  if (my_q < ncopy) {
    const int t = my_q / K;
    const int blk = t / kRouteBlock, tl = t % kRouteBlock;
    const int slot = s_cnt[my_e] + s_pre[blk * N + my_e] +
                     __popcll(sm[blk * N + my_e] & ((1ull << tl) - 1ull));
    slot_of[my_q] = slot;
    token_of[slot] = t;
  }
}

// One workgroup per token; thread c handles 16 bytes of the output row.  The
// Y rows are read once, non-temporally (prefill: 144 -> 136 us per call).  The
// K expert rows are fetched U (8, 16, 24 or 32, the smallest >= K) at a time
// (independent loads in flight) and added in j order.
template <typename T, int U>
__global__ __launch_bounds__(512) void combine_kernel(const T* __restrict__ Y,
                                                      const int32_t* __restrict__ slot_of,
                                                      const float* __restrict__ gate, int K, int l,
                                                      const float* __restrict__ R,
                                                      T* __restrict__ v) {
  constexpr int EPC = 16 / sizeof(T);
  const int t = blockIdx.x;
  const int32_t* so = slot_of + (int64_t)t * K;
  const float* gt = gate + (int64_t)t * K;
  for (int c = threadIdx.x; c * EPC < l; c += blockDim.x) {
    float acc[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < K; j0 += U) {
      // straight-line: rows past K re-read row K-1 and are weighted by zero
      u32x4 y[U];
      float gw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(j0 + u, K - 1);
        y[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Y + (int64_t)so[j] * l + c * EPC));
        gw[u] = j0 + u < K ? gt[j] : 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float gj = gw[u];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += gj * __uint_as_float(y[u][i] << 16);
            acc[2 * i + 1] += gj * __uint_as_float(y[u][i] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += gj * __uint_as_float(y[u][i]);
        }
      }
    }
    if (R != nullptr) {
      const f32x4_t* rr = reinterpret_cast<const f32x4_t*>(R + (int64_t)t * l + c * EPC);
#pragma unroll
      for (int q = 0; q < EPC / 4; ++q) {
        const f32x4_t r4 = rr[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * q + i] += r4[i];
      }
    }
    u32x4 o;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
    }
    *reinterpret_cast<u32x4*>(v + (int64_t)t * l + c * EPC) = o;
  }
}

}  // namespace

bool route_small_fits(int T, int N, int K) {
  return N <= 2048 && (int64_t)((T + kRouteBlock - 1) / kRouteBlock) * N <= kSmallRouteMasks &&
         (int64_t)T * K <= kSmallRouteCopies;
}

template <int NPL>
void launch_topk_npl(const TopkArgs& a, int spl, dim3 grid, int tok_blocks, hipStream_t s) {
  const dim3 block(256);
  if constexpr (NPL * 16 <= 128)
    if (spl == 16) return topk_gate_kernel<NPL, 16><<<grid, block, 0, s>>>(a, tok_blocks);
  if constexpr (NPL * 8 <= 128)
    if (spl == 8) return topk_gate_kernel<NPL, 8><<<grid, block, 0, s>>>(a, tok_blocks);
  if constexpr (NPL * 4 <= 128)
    if (spl == 4) return topk_gate_kernel<NPL, 4><<<grid, block, 0, s>>>(a, tok_blocks);
  if constexpr (NPL * 2 <= 128)
    if (spl == 2) return topk_gate_kernel<NPL, 2><<<grid, block, 0, s>>>(a, tok_blocks);
  topk_gate_kernel<NPL, 1><<<grid, block, 0, s>>>(a, tok_blocks);
}

hipError_t launch_topk_gate(const TopkArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int N = a.N, K = a.K;
  if (N > 64 * kTopkMaxPerLane || K > 64 || K > N || a.lsplits < 1 || !a.logits)
    return hipErrorInvalidValue;
  if (a.u_part && (a.usplits < 1 || a.l <= 0 || a.l % 4 || !a.u || a.u_ld % 4 || a.u_ld < a.l))
    return hipErrorInvalidValue;
  if (a.logits_ld < N || (a.lsplits > 1 && a.logits_sstride < (int64_t)a.T * a.logits_ld))
    return hipErrorInvalidValue;
  const int tok_blocks = (a.T + 3) / 4;
  const int64_t u_blocks = a.u_part ? ((int64_t)a.T * (a.l / 4) + 255) / 256 : 0;
  if (tok_blocks + u_blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(tok_blocks + u_blocks));
  const int npl = (N + 63) / 64;
  // partial sets loaded at once: a power of two >= lsplits, at most 128
  // values per lane
  int spl = a.lsplits <= 1   ? 1
            : a.lsplits <= 2 ? 2
            : a.lsplits <= 4 ? 4
            : a.lsplits <= 8 ? 8
            : a.lsplits <= 16 ? 16 : 1;
  const int npl_c = npl <= 1 ? 1 : npl <= 2 ? 2 : npl <= 4 ? 4 : npl <= 8 ? 8 : npl <= 14 ? 14
                    : npl <= 16 ? 16 : 32;
  if (spl * npl_c > 128) spl = 1;
  switch (npl_c) {
    case 1: launch_topk_npl<1>(a, spl, grid, tok_blocks, s); break;
    case 2: launch_topk_npl<2>(a, spl, grid, tok_blocks, s); break;
    case 4: launch_topk_npl<4>(a, spl, grid, tok_blocks, s); break;
    case 8: launch_topk_npl<8>(a, spl, grid, tok_blocks, s); break;
    case 14: launch_topk_npl<14>(a, spl, grid, tok_blocks, s); break;
    case 16: launch_topk_npl<16>(a, spl, grid, tok_blocks, s); break;
    default: launch_topk_npl<32>(a, spl, grid, tok_blocks, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_route_masks(const int32_t* idx, int T, int N, int K, uint64_t* masks,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int nblk = (T + kRouteBlock - 1) / kRouteBlock;
  route_masks_kernel<<<dim3(nblk), dim3(256), sizeof(uint64_t) * N, s>>>(idx, T, N, K, masks);
  return hipGetLastError();
}

hipError_t launch_route_scan(const uint64_t* masks, int nblk, int N, int tile_m, int32_t* counts,
                             int32_t* offsets, int32_t* base, int32_t* tiles, hipStream_t s,
                             int32_t* active) {
  if (N > 2048 || tile_m <= 0) return hipErrorInvalidValue;
  if (active && (!tiles || tile_m < kActiveTile)) return hipErrorInvalidValue;
  if (N < 1 || nblk < 0) return hipErrorInvalidValue;
  route_colscan_kernel<<<dim3((N + 63) / 64), dim3(1024), 0, s>>>(masks, nblk, N, counts, base);
  route_offsets_kernel<<<dim3(1), dim3(1024), 0, s>>>(counts, N, tile_m, offsets, tiles, active);
  return hipGetLastError();
}

hipError_t launch_route_assign(const int32_t* idx, const uint64_t* masks, const int32_t* base,
                               const int32_t* offsets, int T, int N, int K, int32_t* slot_of,
                               int32_t* token_of, hipStream_t s) {
  const int64_t n = (int64_t)T * K;
  if (n <= 0) return hipSuccess;
  route_assign_kernel<<<dim3((n + 255) / 256), dim3(256), 0, s>>>(idx, masks, base, offsets, T, N, K,
                                                                  slot_of, token_of);
  return hipGetLastError();
}

hipError_t launch_route_small(const int32_t* idx, int T, int N, int K, int tile_m, int32_t* counts,
                              int32_t* offsets, int32_t* tiles, int32_t* slot_of,
                              int32_t* token_of, hipStream_t s, int32_t* active) {
  if (T <= 0) return hipSuccess;
  if (!route_small_fits(T, N, K) || tile_m <= 0) return hipErrorInvalidValue;
  if (active && (!tiles || tile_m < kActiveTile)) return hipErrorInvalidValue;
  const int grid = (T * K + 1023) / 1024;
  route_small_kernel<<<dim3(grid), dim3(1024), 0, s>>>(idx, T, N, K, tile_m, counts, offsets,
                                                       tiles, slot_of, token_of, active);
  return hipGetLastError();
}

template <typename T>
void launch_combine_t(const T* Y, const int32_t* slot_of, const float* gate, int T_, int K, int l,
                      const float* R, T* v, hipStream_t s) {
  // one thread per 16-byte chunk of the row (up to 512 threads, then a
  // loop); as many expert rows in flight as the token has (8, 16, 24 or 32)
  const int chunks = l / (16 / static_cast<int>(sizeof(T)));
  const dim3 grid(T_), block(std::min(512, (chunks + 63) / 64 * 64));
  if (K <= 8) combine_kernel<T, 8><<<grid, block, 0, s>>>(Y, slot_of, gate, K, l, R, v);
  else if (K <= 16) combine_kernel<T, 16><<<grid, block, 0, s>>>(Y, slot_of, gate, K, l, R, v);
  else if (K <= 24) combine_kernel<T, 24><<<grid, block, 0, s>>>(Y, slot_of, gate, K, l, R, v);
  else combine_kernel<T, 32><<<grid, block, 0, s>>>(Y, slot_of, gate, K, l, R, v);
}

hipError_t launch_combine(const void* Y, const int32_t* slot_of, const float* gate, int T, int K,
                          int l, Dt dt, const float* R, void* v, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (R && (reinterpret_cast<uintptr_t>(R) & 15u)) return hipErrorInvalidValue;
  if (dt == Dt::BF16)
    launch_combine_t(static_cast<const uint16_t*>(Y), slot_of, gate, T, K, l, R,
                     static_cast<uint16_t*>(v), s);
  else
    launch_combine_t(static_cast<const float*>(Y), slot_of, gate, T, K, l, R,
                     static_cast<float*>(v), s);
  return hipGetLastError();
}

}  // namespace lmoe
