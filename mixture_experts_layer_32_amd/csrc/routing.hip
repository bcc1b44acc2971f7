// Routing and combine kernels of the LatentMoE layer, for gfx950.
//
// LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in Mixture of
// Experts, §3: routing weights from the router logits, the top-K expert set
// T_{K,N'} of each token, dispatch of the latent token copies to their
// experts and the gate-weighted aggregation sum_{i in T} p'_i E_i(u).
//
//  topk_gate     one wave per token: K rounds of a wave-wide arg-max over
//                (logit desc, expert id asc), then the gate rule.
//  route_masks   per block of 64 tokens, one 64-bit mask per expert of the
//                tokens that chose it (LDS 64-bit atomic OR; integer, exact).
//  route_scan    one workgroup: expert counts = popcounts, exclusive prefix
//                sum over experts (offsets), and the first row of each
//                (block, expert) in the expert-grouped order.
//  route_assign  one thread per copy (t, j): its row is the block base plus
//                the number of earlier tokens of the block that chose the same
//                expert, so rows of an expert follow increasing token index.
//  combine       v[t] = sum_j gate[t][j] * Y[slot_of[t][j]] in fp32, fixed
//                j order (deterministic), rounded once to the output dtype.
#include "common.hpp"
#include "kernels.hpp"

namespace lmoe {
namespace {

constexpr int kTopkMaxPerLane = 32;  // N <= 2048

// fp32 -> uint32 whose unsigned order is the float order (+0 == -0).
__device__ __forceinline__ uint32_t order_key(float z) {
  if (z == 0.f) z = 0.f;
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
    const uint64_t w = (static_cast<uint64_t>(hi) << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ logits,
                                                        const float* __restrict__ bias, int T,
                                                        int N, int K, int gating,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* zr = logits + (int64_t)t * N;

  float z[NPL];
  uint32_t key[NPL];
  uint32_t taken = 0;  // bit i: value i of this lane already selected (or absent)
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = i * 64 + lane;
    if (e < N) {
      z[i] = zr[e] + (bias ? bias[e] : 0.f);
      key[i] = order_key(z[i]);
    } else {
      z[i] = -INFINITY;
      key[i] = 0;
      taken |= 1u << i;
    }
  }

  float my_z = 0.f;
  int my_e = 0;
  for (int j = 0; j < K; ++j) {
    // lane-local best among untaken values; on equal keys the lower expert id
    // (the smaller i, since e = 64 i + lane) wins because of the strict >
    uint64_t best = 0;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const uint64_t kk = (static_cast<uint64_t>(key[i]) << 32) |
                          (0xffffffffu - static_cast<uint32_t>(i * 64 + lane));
      if (!((taken >> i) & 1u) && (bi < 0 || kk > best)) { best = kk; bi = i; }
    }
    const uint64_t win = wave_max_u64(bi < 0 ? 0ull : best);
    const int we = static_cast<int>(0xffffffffu - static_cast<uint32_t>(win));
    if ((we & 63) == lane) {
      const int wi = we >> 6;
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i == wi) taken |= 1u << i;
    }
    // winner's logit, broadcast from its lane
    float wz = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (i == (we >> 6)) wz = z[i];
    wz = __shfl(wz, we & 63, kWave);
    if (lane == j) { my_z = wz; my_e = we; }
  }

  // ---- gates (rule from the layer configuration)
  const bool mine = lane < K;
  const float zmax = __shfl(my_z, 0, kWave);  // first selected = largest logit
  float g = 0.f;
  if (gating == 2) {  // sigmoid, normalised over the selected set
    const float sgm = mine ? 1.f / (1.f + expf(-my_z)) : 0.f;
    const float tot = wave_sum(sgm);
    g = sgm / tot;
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
    idx[(int64_t)t * K + lane] = my_e;
    gate[(int64_t)t * K + lane] = g;
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

// One workgroup of 1024 threads; N <= 2048 (two experts per thread).
// base[b][e] = copies of expert e in routing blocks before b (relative to the
// expert's first row); offsets[e] = rows of all experts before e.
__global__ __launch_bounds__(1024) void route_scan_kernel(const uint64_t* __restrict__ masks,
                                                          int nblk, int N, int tile_m,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ base,
                                                          int32_t* __restrict__ tiles) {
  __shared__ int s_cnt[2048];
  __shared__ int s_til[2048];
  __shared__ int s_wsum[2][16];
  const int tid = threadIdx.x;
  int cnt[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + h * 1024;
    if (e < N) {
      int run = 0;
      int b = 0;
      for (; b + 8 <= nblk; b += 8) {  // 8 independent loads in flight
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = masks[(int64_t)(b + u) * N + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          base[(int64_t)(b + u) * N + e] = run;
          run += __popcll(v[u]);
        }
      }
      for (; b < nblk; ++b) {
        base[(int64_t)b * N + e] = run;
        run += __popcll(masks[(int64_t)b * N + e]);
      }
      cnt[h] = run;
    }
  }
  // exclusive scan over experts of counts and of m-tiles; thread tid owns
  // experts 2*tid and 2*tid+1 of the scan's linear order
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + h * 1024;
    s_cnt[e] = e < N ? cnt[h] : 0;
    s_til[e] = e < N ? (cnt[h] + tile_m - 1) / tile_m : 0;
  }
  __syncthreads();
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
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + h * 1024;
    if (e < N) {
      counts[e] = cnt[h];
      offsets[e] = s_cnt[e];
      if (tiles) tiles[e] = s_til[e];
    }
  }
  if (tid == 0) {
    int total_c = 0, total_t = 0;
    for (int i = 0; i < 16; ++i) { total_c += s_wsum[0][i]; total_t += s_wsum[1][i]; }
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

// One workgroup per token; thread c handles 16 bytes of the output row.
template <typename T>
__global__ __launch_bounds__(128) void combine_kernel(const T* __restrict__ Y,
                                                      const int32_t* __restrict__ slot_of,
                                                      const float* __restrict__ gate, int K, int l,
                                                      T* __restrict__ v) {
  constexpr int EPC = 16 / sizeof(T);
  const int t = blockIdx.x;
  const int32_t* so = slot_of + (int64_t)t * K;
  const float* gt = gate + (int64_t)t * K;
  for (int c = threadIdx.x; c * EPC < l; c += blockDim.x) {
    float acc[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
    for (int j = 0; j < K; ++j) {
      const float gj = gt[j];
      const uint4 y = *reinterpret_cast<const uint4*>(Y + (int64_t)so[j] * l + c * EPC);
      if constexpr (sizeof(T) == 2) {
        const uint32_t w[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += gj * __uint_as_float(w[i] << 16);
          acc[2 * i + 1] += gj * __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
        acc[0] += gj * __uint_as_float(y.x);
        acc[1] += gj * __uint_as_float(y.y);
        acc[2] += gj * __uint_as_float(y.z);
        acc[3] += gj * __uint_as_float(y.w);
      }
    }
    uint4 o;
    if constexpr (sizeof(T) == 2) {
      o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
      o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
      o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
      o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    } else {
      o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                     __float_as_uint(acc[3]));
    }
    *reinterpret_cast<uint4*>(v + (int64_t)t * l + c * EPC) = o;
  }
}

}  // namespace

hipError_t launch_topk_gate(const float* logits, const float* bias, int T, int N, int K,
                            int gating, int32_t* idx, float* gate, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (N > 64 * kTopkMaxPerLane || K > 64 || K > N) return hipErrorInvalidValue;
  const dim3 grid((T + 3) / 4), block(256);
  const int npl = (N + 63) / 64;
  if (npl <= 1) topk_gate_kernel<1><<<grid, block, 0, s>>>(logits, bias, T, N, K, gating, idx, gate);
  else if (npl <= 2) topk_gate_kernel<2><<<grid, block, 0, s>>>(logits, bias, T, N, K, gating, idx, gate);
  else if (npl <= 4) topk_gate_kernel<4><<<grid, block, 0, s>>>(logits, bias, T, N, K, gating, idx, gate);
  else if (npl <= 8) topk_gate_kernel<8><<<grid, block, 0, s>>>(logits, bias, T, N, K, gating, idx, gate);
  else if (npl <= 14) topk_gate_kernel<14><<<grid, block, 0, s>>>(logits, bias, T, N, K, gating, idx, gate);
  else if (npl <= 16) topk_gate_kernel<16><<<grid, block, 0, s>>>(logits, bias, T, N, K, gating, idx, gate);
  else topk_gate_kernel<32><<<grid, block, 0, s>>>(logits, bias, T, N, K, gating, idx, gate);
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
                             int32_t* offsets, int32_t* base, int32_t* tiles, hipStream_t s) {
  if (N > 2048 || tile_m <= 0) return hipErrorInvalidValue;
  route_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(masks, nblk, N, tile_m, counts, offsets, base,
                                                   tiles);
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

hipError_t launch_combine(const void* Y, const int32_t* slot_of, const float* gate, int T, int K,
                          int l, Dt dt, void* v, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dt == Dt::BF16)
    combine_kernel<uint16_t><<<dim3(T), dim3(128), 0, s>>>(static_cast<const uint16_t*>(Y), slot_of,
                                                          gate, K, l, static_cast<uint16_t*>(v));
  else
    combine_kernel<float><<<dim3(T), dim3(128), 0, s>>>(static_cast<const float*>(Y), slot_of, gate,
                                                       K, l, static_cast<float*>(v));
  return hipGetLastError();
}

}  // namespace lmoe
