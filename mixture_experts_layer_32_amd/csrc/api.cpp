// C ABI of the LatentMoE layer forward: validation, workspace planning and
// the stream-ordered launch sequence (include/latentmoe.h).
//
// Layer (LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in
// Mixture of Experts, §3 Eq. (1)/(2)):
//   shared   Hs = sqrelu(x Ws1^T); R = Hs Ws2^T (fp32)   the S shared experts
//   stage 0  u = x W_down^T (bf16/f32 out); logits = r W_r^T (fp32), r = x or u
//   stage 1  top-K per token (ties -> lower id) and gates
//   stage 2  expert histogram / prefix sum / stable row of every token copy
//   stage 3  H = sqrelu(u[token_of] W1_e^T)       grouped by expert
//   stage 4  Y = H W2_e^T                         grouped by expert
//   stage 5  v[t] = sum_j g[t][j] Y[slot_of[t][j]]
//   stage 6  out = v W_up^T + R
// Without projections (standard MoE) stage 0 computes only the logits, the
// expert GEMMs read x, and stage 5 writes `out` directly (adding R there).
// The shared experts read only x: with a side stream (lmoe_overlap) they run
// there, forked at the start of the call and joined before the stage that
// adds R; otherwise they run first on the call's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "latentmoe.h"
#include "kernels.hpp"

struct lmoe_handle {
  lmoe_config cfg;
};

struct lmoe_timer {
  int max_calls = 0;
  int n_calls = 0;
  std::vector<hipEvent_t> ev;  // max_calls * 2 * LMOE_NUM_STAGES: begin and end of each stage
};

struct lmoe_overlap {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

namespace {

thread_local std::string g_last_error;

lmoe_status fail(lmoe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lmoe_status fail(lmoe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

lmoe_status hip_fail(hipError_t e, const char* what) {
  return fail(LMOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxExperts = 2048;
constexpr int64_t kMaxTopK = 64;
constexpr int64_t kMaxShared = 64;
constexpr int64_t kMaxCopies = int64_t(1) << 30;  // T * K (int32 row indices)
// mean copies per expert up to which the streaming kernel beats the tiled one
// (measured on the standard MoE d 4096, m 1536, 128 experts at 32 and 40 rows
// and on latent layers with l 512 and 1024 at 24 to 96 rows: from 48 rows on
// the tiled kernel is as fast or faster)
constexpr double kStreamMaxRowsPerExpert = 40.0;
// fp8 weights: the tiled kernel (one weight tile per expert and 256 columns,
// token rows staged once per tile) from this many rows per expert on
constexpr double kFp8StreamMaxRowsPerExpert = 40.0;
// streaming kernel: passes of 64 rows (4 MFMA row blocks, 128 columns per
// unit) up to this mean row count per expert, of 128 rows (64 columns) above
constexpr double kStreamMb4MaxRowsPerExpert = 40.0;
// fused expert FFN (bf16): up to this many copies per expert on average, so
// that few experts exceed the kernel's 48-row pass
constexpr double kFusedMaxRowsPerExpert = 36.0;
// below this mean row count per expert the streaming kernel works from the
// list of experts with copies (empty experts would otherwise cost a unit
// each: measured 1.7 TB/s at 0.2 rows per expert, 1024 experts)
constexpr double kSparseMaxRowsPerExpert = 2.0;

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Scratch of latentmoe_forward_static, for callers that cannot allocate:
// one copy per device (each GPU the library runs on holds it until the
// process ends).  In host code `scratch` names a host-side stand-in, not
// device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[LMOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

lmoe::Dt act_dt(const lmoe_config& c) { return c.act_dtype == LMOE_F32 ? lmoe::Dt::F32 : lmoe::Dt::BF16; }
lmoe::Dt exp_dt(const lmoe_config& c) {
  return c.expert_dtype == LMOE_F32 ? lmoe::Dt::F32
         : c.expert_dtype == LMOE_BF16 ? lmoe::Dt::BF16
         : c.expert_dtype == LMOE_MXFP4_E2M1 ? lmoe::Dt::MXFP4 : lmoe::Dt::FP8;
}
size_t act_bytes(const lmoe_config& c) { return c.act_dtype == LMOE_F32 ? 4 : 2; }

// Tile config and K split of one dense GEMM (M x N x K).  Large problems:
// the 256 x 256 tile (bf16 operands and output) when it still gives one
// workgroup per compute unit, else 128 x 128 when that gives one (two fit
// per unit); fp32 output with 128 x 128 tiles for at least half the units:
// that tile with K split.  Small problems (decode-sized M): 64 x 64 tiles,
// K split until about two workgroups per compute unit, keeping at least 8 K
// stages per split.
struct DensePlan {
  int tile = 1;
  int splits = 1;
};

constexpr int64_t kComputeUnits = 256;  // MI355X

DensePlan plan_dense(int64_t M, int64_t N, int64_t K, size_t elem_bytes, bool bf16_out) {
  DensePlan d;
  if (M <= 0 || N <= 0 || K <= 0) return d;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (elem_bytes == 2 && bf16_out && t256 >= kComputeUnits) {
    d.tile = 2;
    return d;
  }
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= kComputeUnits) {
    d.tile = 0;
    return d;
  }
  const int64_t stages = (K * int64_t(elem_bytes) + 127) / 128;
  if (!bf16_out && 2 * t128 >= kComputeUnits) {
    // fp32 output (partials that the consumer adds), 128 x 128 tiles short of
    // one per compute unit: split K to the count that minimises waves x
    // stages per split at two workgroups per unit (the fewest splits on a
    // tie), at most 4 (every partial set is written once and read once);
    // the 64 x 64 tile reads twice the operand bytes per flop here
    d.tile = 0;
    int64_t best = -1;
    for (int64_t s = 1; s <= 4 && (s == 1 || stages / s >= 8); ++s) {
      const int64_t waves = (t128 * s + 2 * kComputeUnits - 1) / (2 * kComputeUnits);
      const int64_t cost = waves * ((stages + s - 1) / s);
      if (best < 0 || cost < best) { best = cost; d.splits = static_cast<int>(s); }
    }
    if (N % 4) d.splits = 1;
    return d;
  }
  d.tile = 1;
  const int64_t small = ((M + 63) / 64) * ((N + 63) / 64);
  int64_t s = (2 * kComputeUnits + small - 1) / small;
  s = std::min<int64_t>(s, std::max<int64_t>(1, stages / 8));
  if (N % 4) s = 1;
  d.splits = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, 16)));
  return d;
}

// Dense GEMM on 128 x 128 tiles with K split until about `per_cu` workgroups
// per compute unit (at least 8 K stages per split, at most 16 splits).  Fewer
// operand bytes per flop than the 64 x 64 tile for decode-sized M.
DensePlan plan_dense_128(int64_t M, int64_t N, int64_t K, size_t elem_bytes, int per_cu) {
  DensePlan d;
  d.tile = 0;
  if (M <= 0 || N <= 0 || K <= 0) return d;
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t stages = (K * int64_t(elem_bytes) + 127) / 128;
  int64_t s = (per_cu * kComputeUnits + t128 - 1) / t128;
  s = std::min<int64_t>(s, std::max<int64_t>(1, stages / 8));
  if (N % 4) s = 1;
  d.splits = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, 16)));
  return d;
}

// Shared-expert GEMMs: 128 x 128 tiles, one workgroup per compute unit
// (plan_dense_128's mode 1)
constexpr int kSharedPlan = 1;

// Tile of the grouped expert GEMMs when experts receive many tokens: 128 rows
// keeps the padding of each expert's last tile small, 256 columns halve the
// operand bytes per flop against 128 x 128.
constexpr int kExpertTile = 3;
// experts with many rows (prefill): 256 x 256 tiles (the persistent grouped
// kernel for bf16 layers) from this mean row count per expert on (at 48 rows
// their padding would waste work)
constexpr double kBigTileRowsPerExpert = 256.0;

struct Plan {
  int64_t T = 0, copies = 0;
  int nblk = 0;
  bool stream = true;   // expert GEMMs: weight-streaming kernel
  bool sparse = false;  // streaming kernel over the list of experts with copies only
  bool fused = false;   // FC1 + FC2 in the fused weight-streaming kernel
  bool grouped = false; // expert GEMMs in the persistent grouped kernel (prefill)
  int mb_max = 4;       // streaming kernel rows per pass / 16
  int expert_tile = 0;  // tiled kernel tile config
  int tile_m = 128;
  DensePlan down, router, up;
  // W_down / W_up in the persistent grouped kernel as one group of T rows
  // (bf16, 256 x 256 tiles, at least one tile per compute unit, no residual)
  bool down_grouped = false, up_grouped = false;
  // split-K partials left for the top-k kernel to add: the router logits,
  // and the down-projection when the router reads x (nothing needs u before)
  bool defer_u = false, defer_z = false;
  size_t part_z = 0;    // byte offset of the router partials in the partial region
  // router on x with split K: W_down and W_r in one launch over x (output
  // columns 0..l-1 from W_down, l..l+N-1 from W_r), partials only
  bool front = false;
  DensePlan front_plan;
  DensePlan sh1, sh2;   // shared experts: x Ws1^T (+ sqrelu), Hs Ws2^T (fp32 out)
  size_t u, ublk, logits, idx, gate, masks, base, counts, offsets, tiles, slot, token, H, Y, v,
      partial, Hs, R, partial_sh, active, total;
};

Plan make_plan(const lmoe_config& c, int64_t T) {
  Plan p;
  p.T = T;
  p.copies = T * c.top_k;
  p.nblk = static_cast<int>((T + lmoe::kRouteBlock - 1) / lmoe::kRouteBlock);
  const double mean = T > 0 ? double(p.copies) / double(c.n_experts) : 0.0;
  const bool fp8 = c.expert_dtype == LMOE_FP8_E4M3_ROWSCALE;
  const bool fp4 = c.expert_dtype == LMOE_MXFP4_E2M1;
  const bool bf16 = c.act_dtype == LMOE_BF16 && c.expert_dtype == LMOE_BF16;
  switch (c.expert_kernel) {
    case LMOE_EXPERTS_TILED: p.stream = false; break;
    case LMOE_EXPERTS_STREAM: p.stream = true; break;
    case LMOE_EXPERTS_FUSED: p.stream = p.fused = true; break;
    default:
      p.stream = fp8 ? mean <= kFp8StreamMaxRowsPerExpert : mean <= kStreamMaxRowsPerExpert;
      // one expert per resident workgroup: the fused kernel fills the chip
      // only with at least one expert per compute unit (bf16 or MXFP4
      // weights, bf16 tokens)
      p.fused = p.stream && (bf16 || (fp4 && c.act_dtype == LMOE_BF16)) &&
                mean <= kFusedMaxRowsPerExpert &&
                lmoe::ffn_stream_fits(static_cast<int>(c.n_experts), static_cast<int>(c.l),
                                      static_cast<int>(c.m), c.activation == LMOE_ACT_SWIGLU,
                                      fp4) &&
                c.n_experts >= kComputeUnits;
  }
  if (fp4 && !p.stream) p.stream = true;  // MXFP4 weights: no tiled kernel
  p.mb_max = mean <= kStreamMb4MaxRowsPerExpert ? 4 : 8;
  // most experts empty (expected share e^-mean > 1/8): the streaming kernel
  // visits only the experts with copies, listed by the dispatch stage
  p.sparse = p.stream && !p.fused && mean < kSparseMaxRowsPerExpert;
  p.expert_tile = c.act_dtype == LMOE_BF16 ? (mean >= kBigTileRowsPerExpert ? 2 : kExpertTile)
                                           : 1;  // fp32: the 64 x 64 tile
  p.tile_m = fp8 ? lmoe::fp8w_block_m() : lmoe::tiled_block_m(p.expert_tile);
  {
    // many rows per expert, bf16: the persistent grouped kernel (mixed tile
    // heights, so skewed loads pad little) for both expert GEMMs
    const int n1 = static_cast<int>(c.activation == LMOE_ACT_SWIGLU ? 2 * c.m : c.m);
    p.grouped = !p.stream && bf16 && mean >= kBigTileRowsPerExpert &&
                lmoe::gemm_grouped_fits(n1, static_cast<int>(c.l), static_cast<int>(c.n_experts)) &&
                lmoe::gemm_grouped_fits(static_cast<int>(c.l), static_cast<int>(c.m),
                                        static_cast<int>(c.n_experts));
  }
  const size_t ab = act_bytes(c);
  const int64_t r_in = c.router_input == LMOE_ROUTER_ON_LATENT ? c.l : c.d;
  size_t partial = 0;
  if (c.has_projections) {
    p.down = plan_dense(T, c.l, c.d, ab, ab == 2);
    p.up = plan_dense(T, c.d, c.l, ab, ab == 2);
    partial = std::max(partial, size_t(p.down.splits > 1 ? p.down.splits : 0) * T * c.l * 4);
    partial = std::max(partial, size_t(p.up.splits > 1 ? p.up.splits : 0) * T * c.d * 4);
  }
  p.router = plan_dense(T, c.n_experts, r_in, ab, false);  // fp32 logits
  if (c.has_projections && ab == 2) {
    const auto tiles256 = [&](int64_t n) { return ((T + 255) / 256) * (n / 256); };
    p.down_grouped = p.down.tile == 2 && p.down.splits == 1 &&
                     lmoe::gemm_grouped_fits(static_cast<int>(c.l), static_cast<int>(c.d), 1) &&
                     tiles256(c.l) >= kComputeUnits;
    p.up_grouped = p.up.tile == 2 && p.up.splits == 1 && c.n_shared == 0 &&
                   lmoe::gemm_grouped_fits(static_cast<int>(c.d), static_cast<int>(c.l), 1) &&
                   tiles256(c.d) >= kComputeUnits;
  }
  p.defer_u = c.has_projections && c.router_input == LMOE_ROUTER_ON_X && p.down.splits > 1;
  p.defer_z = p.router.splits > 1;
  if (p.defer_u && p.defer_z) {
    p.front_plan = plan_dense(T, c.l + c.n_experts, c.d, ab, false);
    const int bn = p.front_plan.tile == 1 ? 64 : 128;  // column tile of plan_dense's tiles 0 / 1
    p.front = p.front_plan.splits > 1 && p.front_plan.tile <= 1 && c.l % bn == 0;
    if (p.front && p.front_plan.tile == 1) {
      // about three 64 x 64 split tiles per compute unit (measured best for
      // the decode shapes: one launch over x for both weight matrices)
      const int64_t small = ((T + 63) / 64) * ((c.l + c.n_experts + 63) / 64);
      const int64_t stages = (c.d * int64_t(ab) + 127) / 128;
      int64_t sp = (3 * kComputeUnits + small - 1) / small;
      sp = std::min<int64_t>({sp, std::max<int64_t>(2, stages / 8), 16});
      p.front_plan.splits = static_cast<int>(std::max<int64_t>(2, sp));
    }
    if (p.front)
      partial = std::max(partial, size_t(p.front_plan.splits) * T * (c.l + c.n_experts) * 4);
  }
  const size_t router_part = size_t(p.router.splits > 1 ? p.router.splits : 0) * T * c.n_experts * 4;
  if (p.defer_u) {  // both partial sets live until the top-k kernel
    p.part_z = align_up(size_t(p.down.splits) * T * c.l * 4);
    partial = std::max(partial, p.part_z + router_part);
  } else {
    partial = std::max(partial, router_part);
  }
  // shared experts: their own partial region (they may run beside the routed path)
  const int64_t hs = c.n_shared * c.m_shared;
  size_t partial_sh = 0;
  // SwiGLU: the shared FC1 computes 2 * hs columns (up, gate pairs)
  const int64_t hs1 = c.activation == LMOE_ACT_SWIGLU ? 2 * hs : hs;
  if (hs > 0) {
    if (ab != 2) {
      p.sh1 = plan_dense(T, hs1, c.d, ab, ab == 2);
      p.sh2 = plan_dense(T, c.d, hs, ab, false);
    } else {
      p.sh1 = plan_dense_128(T, hs1, c.d, ab, kSharedPlan);
      p.sh2 = plan_dense_128(T, c.d, hs, ab, kSharedPlan);
      const int64_t t256 = ((T + 255) / 256) * ((hs1 + 255) / 256);
      if (t256 >= kComputeUnits) p.sh1 = plan_dense(T, hs1, c.d, ab, true);
    }
    partial_sh = std::max(size_t(p.sh1.splits > 1 ? p.sh1.splits : 0) * T * hs1 * 4,
                          size_t(p.sh2.splits > 1 ? p.sh2.splits : 0) * T * c.d * 4);
  }
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  p.u = take(c.has_projections ? size_t(T) * c.l * ab : 0);
  // grouped regime: u (or x) in 32-column blocks over all T rows, which
  // FC1 gathers from (consecutive tokens of an expert then lie side by side)
  p.ublk = take(p.grouped ? size_t(T) * c.l * ab : 0);
  p.logits = take(size_t(T) * c.n_experts * 4);
  p.idx = take(size_t(p.copies) * 4);
  p.gate = take(size_t(p.copies) * 4);
  p.masks = take(size_t(p.nblk) * c.n_experts * 8);
  p.base = take(size_t(p.nblk) * c.n_experts * 4);
  p.counts = take(size_t(c.n_experts) * 4);
  p.offsets = take(size_t(c.n_experts + 1) * 4);
  p.tiles = take(size_t(c.n_experts + 1) * 4);
  p.slot = take(size_t(p.copies) * 4);
  p.token = take(size_t(p.copies) * 4);
  p.H = take(p.fused ? 0 : size_t(p.copies) * c.m * ab);  // the fused kernel keeps H on chip
  p.Y = take(size_t(p.copies) * c.l * ab);
  p.v = take(c.has_projections ? size_t(T) * c.l * ab : 0);
  p.partial = take(partial);
  p.Hs = take(size_t(T) * hs * ab);
  p.R = take(hs > 0 ? size_t(T) * c.d * 4 : 0);
  p.partial_sh = take(partial_sh);
  p.active = take(size_t(c.n_experts) * 4);
  p.total = o;
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char* latentmoe_status_string(lmoe_status s) {
  switch (s) {
    case LMOE_OK: return "ok";
    case LMOE_ERR_INVALID_ARG: return "invalid argument";
    case LMOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case LMOE_ERR_WORKSPACE: return "workspace missing or too small";
    case LMOE_ERR_HIP: return "HIP runtime error";
    case LMOE_ERR_ALLOC: return "host allocation failed";
  }
  return "unknown status";
}

const char* latentmoe_last_error(void) { return g_last_error.c_str(); }

lmoe_status latentmoe_create(const lmoe_config* cfg, lmoe_handle** out) {
  if (!cfg || !out) return fail(LMOE_ERR_INVALID_ARG, "create: NULL argument");
  *out = nullptr;
  const lmoe_config& c = *cfg;
  if (c.d <= 0 || c.l <= 0 || c.m <= 0 || c.n_experts <= 0 || c.top_k <= 0)
    return fail(LMOE_ERR_INVALID_ARG, "create: sizes must be positive");
  if (c.top_k > c.n_experts)
    return fail(LMOE_ERR_INVALID_ARG, "create: top_k %lld > n_experts %lld", (long long)c.top_k,
                (long long)c.n_experts);
  if (c.has_projections != 0 && c.has_projections != 1)
    return fail(LMOE_ERR_INVALID_ARG, "create: has_projections must be 0 or 1");
  if (!c.has_projections && c.l != c.d)
    return fail(LMOE_ERR_INVALID_ARG, "create: without projections l must equal d");
  if (c.has_projections && c.l > c.d)
    return fail(LMOE_ERR_INVALID_ARG, "create: latent width l > d");
  if (c.router_input != LMOE_ROUTER_ON_X && c.router_input != LMOE_ROUTER_ON_LATENT)
    return fail(LMOE_ERR_INVALID_ARG, "create: bad router_input");
  if (c.gating < LMOE_GATE_SOFTMAX_ALL || c.gating > LMOE_GATE_SIGMOID_TOPK_NORM)
    return fail(LMOE_ERR_INVALID_ARG, "create: bad gating");
  if (c.has_router_bias != 0 && c.has_router_bias != 1)
    return fail(LMOE_ERR_INVALID_ARG, "create: has_router_bias must be 0 or 1");
  if (c.activation != LMOE_ACT_SQRELU && c.activation != LMOE_ACT_SWIGLU)
    return fail(LMOE_ERR_INVALID_ARG, "create: bad activation");
  if (c.act_dtype < LMOE_F32 || c.act_dtype > LMOE_MXFP4_E2M1 ||
      c.expert_dtype < LMOE_F32 || c.expert_dtype > LMOE_MXFP4_E2M1)
    return fail(LMOE_ERR_INVALID_ARG, "create: bad dtype");
  const bool ok_pair = (c.act_dtype == LMOE_F32 && c.expert_dtype == LMOE_F32) ||
                       (c.act_dtype == LMOE_BF16 && c.expert_dtype == LMOE_BF16) ||
                       (c.act_dtype == LMOE_BF16 && c.expert_dtype == LMOE_FP8_E4M3_ROWSCALE) ||
                       (c.act_dtype == LMOE_BF16 && c.expert_dtype == LMOE_MXFP4_E2M1);
  if (!ok_pair)
    return fail(LMOE_ERR_UNSUPPORTED, "create: dtype pair (act %d, experts %d) not implemented",
                c.act_dtype, c.expert_dtype);
  if (c.d % 16 || c.l % 16 || c.m % 16)
    return fail(LMOE_ERR_UNSUPPORTED, "create: d, l, m must be multiples of 16");
  if (c.n_experts > kMaxExperts || c.top_k > kMaxTopK)
    return fail(LMOE_ERR_UNSUPPORTED, "create: n_experts <= %lld and top_k <= %lld supported",
                (long long)kMaxExperts, (long long)kMaxTopK);
  if (c.d > (int64_t(1) << 20) || c.m > (int64_t(1) << 20))
    return fail(LMOE_ERR_UNSUPPORTED, "create: widths above 2^20");
  if (c.expert_kernel < LMOE_EXPERTS_AUTO || c.expert_kernel > LMOE_EXPERTS_FUSED)
    return fail(LMOE_ERR_INVALID_ARG, "create: bad expert_kernel");
  if (c.expert_dtype == LMOE_MXFP4_E2M1) {
    if (c.l % 32 || c.m % 32)
      return fail(LMOE_ERR_UNSUPPORTED, "create: MXFP4 experts need l and m multiples of 32");
    if (c.expert_kernel == LMOE_EXPERTS_TILED)
      return fail(LMOE_ERR_UNSUPPORTED, "create: MXFP4 experts run in the streaming or fused kernels");
  }
  if (c.n_shared < 0 || (c.n_shared > 0 && c.m_shared <= 0))
    return fail(LMOE_ERR_INVALID_ARG, "create: n_shared < 0, or shared experts without a width");
  if (c.n_shared > kMaxShared || (c.n_shared > 0 && (c.m_shared % 16 || c.m_shared > (int64_t(1) << 20))))
    return fail(LMOE_ERR_UNSUPPORTED, "create: n_shared <= %lld and m_shared a multiple of 16 "
                "up to 2^20 supported", (long long)kMaxShared);
  if (c.expert_kernel == LMOE_EXPERTS_FUSED &&
      !(c.act_dtype == LMOE_BF16 &&
        (c.expert_dtype == LMOE_BF16 || c.expert_dtype == LMOE_MXFP4_E2M1) &&
        lmoe::ffn_stream_fits(static_cast<int>(c.n_experts), static_cast<int>(c.l),
                              static_cast<int>(c.m), c.activation == LMOE_ACT_SWIGLU,
                              c.expert_dtype == LMOE_MXFP4_E2M1)))
    return fail(LMOE_ERR_UNSUPPORTED,
                "create: the fused expert kernel needs bf16 activations, bf16 or MXFP4 experts, "
                "m <= 1536 and each expert weight array below 2 GiB");
  lmoe_handle* h = new (std::nothrow) lmoe_handle;
  if (!h) return fail(LMOE_ERR_ALLOC, "create: out of host memory");
  h->cfg = c;
  *out = h;
  return LMOE_OK;
}

lmoe_status latentmoe_destroy(lmoe_handle* h) {
  delete h;
  return LMOE_OK;
}

lmoe_status latentmoe_workspace_size(const lmoe_handle* h, int64_t T, size_t* bytes) {
  if (!h || !bytes) return fail(LMOE_ERR_INVALID_ARG, "workspace_size: NULL argument");
  if (T < 0) return fail(LMOE_ERR_INVALID_ARG, "workspace_size: T < 0");
  if (T * h->cfg.top_k > kMaxCopies) return fail(LMOE_ERR_UNSUPPORTED, "workspace_size: T*K too large");
  *bytes = make_plan(h->cfg, T).total;
  return LMOE_OK;
}

namespace {
// Band height of the packed expert weights: 256 rows (bf16, the grouped
// kernel's weight tile) or 16 (fp8, one n-block of the fp8 kernel); 0 = no
// packed copy for this layer
int packed_band_rows(const lmoe_config& c) {
  if (c.act_dtype != LMOE_BF16) return 0;
  const int64_t n1 = c.activation == LMOE_ACT_SWIGLU ? 2 * c.m : c.m;
  const int G = static_cast<int>(c.n_experts);
  if (c.expert_dtype == LMOE_BF16)
    return lmoe::gemm_grouped_fits(static_cast<int>(n1), static_cast<int>(c.l), G) &&
                   lmoe::gemm_grouped_fits(static_cast<int>(c.l), static_cast<int>(c.m), G)
               ? 256 : 0;
  if (c.expert_dtype == LMOE_FP8_E4M3_ROWSCALE)
    return lmoe::gemm_fp8w_fits(static_cast<int>(n1), static_cast<int>(c.l), G) &&
                   lmoe::gemm_fp8w_fits(static_cast<int>(c.l), static_cast<int>(c.m), G) &&
                   c.l % 64 == 0 && c.m % 64 == 0
               ? 16 : 0;
  return 0;
}
size_t packed_elem_bytes(const lmoe_config& c) {
  return c.expert_dtype == LMOE_FP8_E4M3_ROWSCALE ? 1 : 2;
}
}  // namespace

size_t latentmoe_packed_weights_size(const lmoe_handle* h) {
  if (!h || packed_band_rows(h->cfg) == 0) return 0;
  const lmoe_config& c = h->cfg;
  const int64_t n1 = c.activation == LMOE_ACT_SWIGLU ? 2 * c.m : c.m;
  return size_t(c.n_experts) * size_t(n1 * c.l + c.l * c.m) * packed_elem_bytes(c);
}

lmoe_status latentmoe_pack_expert_weights(const lmoe_handle* h, const lmoe_weights* w, void* packed,
                                          size_t packed_bytes, void* stream) {
  if (!h || !w || !packed) return fail(LMOE_ERR_INVALID_ARG, "pack_expert_weights: NULL argument");
  const size_t need = latentmoe_packed_weights_size(h);
  if (need == 0)
    return fail(LMOE_ERR_UNSUPPORTED, "pack_expert_weights: this layer's experts do not run in the "
                "grouped kernel");
  if (packed_bytes < need)
    return fail(LMOE_ERR_WORKSPACE, "pack_expert_weights: %zu bytes < required %zu", packed_bytes, need);
  if (!w->w1 || !w->w2) return fail(LMOE_ERR_INVALID_ARG, "pack_expert_weights: NULL w1 or w2");
  if (!aligned16(w->w1) || !aligned16(w->w2) || !aligned16(packed))
    return fail(LMOE_ERR_INVALID_ARG, "pack_expert_weights: pointers must be 16-byte aligned");
  const lmoe_config& c = h->cfg;
  const int N = static_cast<int>(c.n_experts), l = static_cast<int>(c.l), m = static_cast<int>(c.m);
  const int n1 = c.activation == LMOE_ACT_SWIGLU ? 2 * m : m;
  const int eb = static_cast<int>(packed_elem_bytes(c)), R = packed_band_rows(c);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* dst = static_cast<char*>(packed);
  hipError_t e = lmoe::launch_pack_bands(w->w1, dst, N, n1, l * eb, R, s);
  if (e != hipSuccess) return hip_fail(e, "pack W1");
  e = lmoe::launch_pack_bands(w->w2, dst + size_t(N) * n1 * l * eb, N, l, m * eb, R, s);
  if (e != hipSuccess) return hip_fail(e, "pack W2");
  return LMOE_OK;
}

const char* latentmoe_expert_regime(const lmoe_handle* h, int64_t T) {
  if (!h || T < 0) return "invalid";
  const Plan p = make_plan(h->cfg, T);
  if (p.fused || p.stream) return p.fused ? "fused" : "stream";
  if (p.grouped) return "grouped";
  return h->cfg.expert_dtype == LMOE_FP8_E4M3_ROWSCALE ? "fp8w" : "tiled";
}

lmoe_status latentmoe_timer_create(lmoe_timer** out) {
  if (!out) return fail(LMOE_ERR_INVALID_ARG, "timer_create: NULL argument");
  lmoe_timer* t = new (std::nothrow) lmoe_timer;
  if (!t) return fail(LMOE_ERR_ALLOC, "timer_create: out of host memory");
  t->max_calls = 256;
  t->ev.assign(size_t(t->max_calls) * 2 * LMOE_NUM_STAGES, nullptr);
  for (auto& e : t->ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      for (auto& f : t->ev)
        if (f) (void)hipEventDestroy(f);
      delete t;
      return hip_fail(r, "timer_create: hipEventCreate");
    }
  }
  *out = t;
  return LMOE_OK;
}

lmoe_status latentmoe_timer_read(lmoe_timer* t, float* stage_ms, int32_t n_stages, int32_t* n_calls) {
  if (!t || !stage_ms || n_stages < LMOE_NUM_STAGES)
    return fail(LMOE_ERR_INVALID_ARG, "timer_read: bad argument");
  for (int s = 0; s < n_stages; ++s) stage_ms[s] = 0.f;
  const int n = t->n_calls;
  for (int c = 0; c < n; ++c) {
    // stage s of call c: events 2s (begin) and 2s + 1 (end), possibly on
    // the side stream (shared experts)
    const hipEvent_t* e = &t->ev[size_t(c) * 2 * LMOE_NUM_STAGES];
    for (int s = 0; s < LMOE_NUM_STAGES; ++s) {
      hipError_t r = hipEventSynchronize(e[2 * s + 1]);
      if (r != hipSuccess) return hip_fail(r, "timer_read: hipEventSynchronize");
      float ms = 0.f;
      r = hipEventElapsedTime(&ms, e[2 * s], e[2 * s + 1]);
      if (r != hipSuccess) return hip_fail(r, "timer_read: hipEventElapsedTime");
      stage_ms[s] += ms;
    }
  }
  if (n_calls) *n_calls = n;
  t->n_calls = 0;
  return LMOE_OK;
}

lmoe_status latentmoe_timer_destroy(lmoe_timer* t) {
  if (!t) return LMOE_OK;
  for (auto& e : t->ev)
    if (e) (void)hipEventDestroy(e);
  delete t;
  return LMOE_OK;
}

lmoe_status latentmoe_overlap_create(void* side_stream, lmoe_overlap** out) {
  if (!out) return fail(LMOE_ERR_INVALID_ARG, "overlap_create: NULL argument");
  *out = nullptr;
  if (!side_stream) return fail(LMOE_ERR_INVALID_ARG, "overlap_create: the side stream must not be NULL");
  lmoe_overlap* o = new (std::nothrow) lmoe_overlap;
  if (!o) return fail(LMOE_ERR_ALLOC, "overlap_create: out of host memory");
  o->side = static_cast<hipStream_t>(side_stream);
  hipError_t r = hipEventCreateWithFlags(&o->fork, hipEventDisableTiming);
  if (r == hipSuccess) r = hipEventCreateWithFlags(&o->join, hipEventDisableTiming);
  if (r != hipSuccess) {
    if (o->fork) (void)hipEventDestroy(o->fork);
    delete o;
    return hip_fail(r, "overlap_create: hipEventCreateWithFlags");
  }
  *out = o;
  return LMOE_OK;
}

lmoe_status latentmoe_overlap_destroy(lmoe_overlap* o) {
  if (!o) return LMOE_OK;
  (void)hipEventDestroy(o->fork);
  (void)hipEventDestroy(o->join);
  delete o;
  return LMOE_OK;
}

lmoe_status latentmoe_forward(const lmoe_handle* h, const lmoe_weights* w, const void* x,
                              int64_t T, void* out, const lmoe_debug_out* dbg, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return latentmoe_forward_overlap(h, w, x, T, out, dbg, workspace, workspace_bytes, stream, nullptr);
}

lmoe_status latentmoe_forward_overlap(const lmoe_handle* h, const lmoe_weights* w, const void* x,
                                      int64_t T, void* out, const lmoe_debug_out* dbg,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      lmoe_overlap* ov) {
  if (!h || !w) return fail(LMOE_ERR_INVALID_ARG, "forward: NULL handle or weights");
  if (T < 0) return fail(LMOE_ERR_INVALID_ARG, "forward: T < 0");
  if (T == 0) return LMOE_OK;
  const lmoe_config& c = h->cfg;
  if (T * c.top_k > kMaxCopies) return fail(LMOE_ERR_UNSUPPORTED, "forward: T*K too large");
  if (!x || !out) return fail(LMOE_ERR_INVALID_ARG, "forward: NULL x or out");
  if (!w->w_router || !w->w1 || !w->w2)
    return fail(LMOE_ERR_INVALID_ARG, "forward: NULL router or expert weights");
  if (c.has_projections && (!w->w_down || !w->w_up))
    return fail(LMOE_ERR_INVALID_ARG, "forward: NULL projection weights");
  if (c.has_router_bias && !w->router_bias)
    return fail(LMOE_ERR_INVALID_ARG, "forward: NULL router bias");
  if (c.expert_dtype == LMOE_FP8_E4M3_ROWSCALE && (!w->w1_scale || !w->w2_scale))
    return fail(LMOE_ERR_INVALID_ARG, "forward: NULL fp8 scales");
  if (c.expert_dtype == LMOE_MXFP4_E2M1 && (!w->w1_mx || !w->w2_mx))
    return fail(LMOE_ERR_INVALID_ARG, "forward: NULL MXFP4 block scales");
  const bool shared = c.n_shared > 0;
  if (shared && (!w->w_shared1 || !w->w_shared2))
    return fail(LMOE_ERR_INVALID_ARG, "forward: NULL shared-expert weights");
  if (ov && static_cast<hipStream_t>(stream) == ov->side)
    return fail(LMOE_ERR_INVALID_ARG, "forward: the side stream must differ from the call's stream");
  const void* ptrs[] = {x, out, w->w_router, w->w1, w->w2, w->w_down, w->w_up,
                        shared ? w->w_shared1 : nullptr, shared ? w->w_shared2 : nullptr,
                        w->experts_packed};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(LMOE_ERR_INVALID_ARG, "forward: pointers must be 16-byte aligned");
  const Plan p = make_plan(c, T);
  if (!workspace || workspace_bytes < p.total)
    return fail(LMOE_ERR_WORKSPACE, "forward: workspace %zu bytes < required %zu", workspace_bytes,
                p.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(LMOE_ERR_INVALID_ARG, "forward: workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  // expert FC1: squared ReLU, or SwiGLU over interleaved (up, gate) weight rows
  const bool glu = c.activation == LMOE_ACT_SWIGLU;
  const int act1 = glu ? lmoe::kActSwiGlu : lmoe::kActSqRelu;
  const lmoe::Dt adt = act_dt(c), edt = exp_dt(c);
  const int ab = static_cast<int>(act_bytes(c));
  const int Ti = static_cast<int>(T), N = static_cast<int>(c.n_experts), K = static_cast<int>(c.top_k);
  const int d = static_cast<int>(c.d), l = static_cast<int>(c.l), m = static_cast<int>(c.m);

  void* u = c.has_projections ? ws + p.u : const_cast<void*>(x);
  float* logits = reinterpret_cast<float*>(ws + p.logits);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + p.idx);
  float* gate = reinterpret_cast<float*>(ws + p.gate);
  uint64_t* masks = reinterpret_cast<uint64_t*>(ws + p.masks);
  int32_t* base = reinterpret_cast<int32_t*>(ws + p.base);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + p.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + p.offsets);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + p.tiles);
  int32_t* slot_of = reinterpret_cast<int32_t*>(ws + p.slot);
  int32_t* token_of = reinterpret_cast<int32_t*>(ws + p.token);
  int32_t* active = p.sparse ? reinterpret_cast<int32_t*>(ws + p.active) : nullptr;
  const int route_tile = p.sparse ? lmoe::kActiveTile : p.tile_m;
  void* H = ws + p.H;
  void* Y = ws + p.Y;
  void* v = c.has_projections ? ws + p.v : out;
  float* partial = reinterpret_cast<float*>(ws + p.partial);
  void* Hs = ws + p.Hs;
  float* R = shared ? reinterpret_cast<float*>(ws + p.R) : nullptr;
  float* partial_sh = reinterpret_cast<float*>(ws + p.partial_sh);

  lmoe_timer* tm = dbg ? dbg->timer : nullptr;
  hipEvent_t* ev = nullptr;
  if (tm) {
    if (tm->n_calls >= tm->max_calls)
      return fail(LMOE_ERR_INVALID_ARG, "forward: timer full (%d calls); read it first", tm->max_calls);
    ev = &tm->ev[size_t(tm->n_calls) * 2 * LMOE_NUM_STAGES];
    ++tm->n_calls;
  }
  hipError_t e;
#define LMOE_TRY(call, what)                          \
  do {                                                \
    e = (call);                                       \
    if (e != hipSuccess) return hip_fail(e, what);    \
  } while (0)
  // stage i: begin / end events (stages 0..6 follow each other on `s`)
#define LMOE_BEGIN(i, st) \
  if (ev) LMOE_TRY(hipEventRecord(ev[2 * (i)], st), "hipEventRecord")
#define LMOE_END(i, st) \
  if (ev) LMOE_TRY(hipEventRecord(ev[2 * (i) + 1], st), "hipEventRecord")
#define LMOE_MARK(i) \
  if (ev) {                                                                  \
    if ((i) > 0) LMOE_TRY(hipEventRecord(ev[2 * (i) - 1], s), "hipEventRecord"); \
    if ((i) < LMOE_STAGE_SHARED) LMOE_TRY(hipEventRecord(ev[2 * (i)], s), "hipEventRecord"); \
  }

  // ---- shared experts (second sum of Eq. (1)/(2)), on x only: on the side
  // stream after a fork from `s`, or first on `s`
  hipStream_t ss = ov && shared ? ov->side : s;
  if (ss != s) {
    LMOE_TRY(hipEventRecord(ov->fork, s), "hipEventRecord (fork)");
    LMOE_TRY(hipStreamWaitEvent(ss, ov->fork, 0), "hipStreamWaitEvent (fork)");
  }
  LMOE_BEGIN(LMOE_STAGE_SHARED, ss);
  if (shared) {
    const int hs = static_cast<int>(c.n_shared * c.m_shared);
    lmoe::GemmArgs a;
    a.A = x; a.lda = d; a.B = w->w_shared1; a.ldb = d; a.C = Hs; a.ldc = hs;
    a.M = Ti; a.N = glu ? 2 * hs : hs; a.K = d; a.act = act1;
    LMOE_TRY(lmoe::launch_gemm_tiled(a, adt, adt, p.sh1.tile, ss, p.sh1.splits, partial_sh),
             "shared FC1 GEMM");
    lmoe::GemmArgs b;
    b.A = Hs; b.lda = hs; b.B = w->w_shared2; b.ldb = hs; b.C = R; b.ldc = d;
    b.M = Ti; b.N = d; b.K = hs;
    LMOE_TRY(lmoe::launch_gemm_tiled(b, adt, lmoe::Dt::F32, p.sh2.tile, ss, p.sh2.splits, partial_sh),
             "shared FC2 GEMM");
  }
  LMOE_END(LMOE_STAGE_SHARED, ss);
  if (ss != s) LMOE_TRY(hipEventRecord(ov->join, ss), "hipEventRecord (join)");
  // the stage that adds R waits for the side stream
  auto join = [&]() -> hipError_t {
    return ss != s ? hipStreamWaitEvent(s, ov->join, 0) : hipSuccess;
  };

  LMOE_MARK(0);
  // ---- stage 0: down-projection and router logits (split-K partials that
  // the top-k kernel adds when deferred)
  float* part_z = reinterpret_cast<float*>(ws + p.partial + p.part_z);
  const int64_t front_ld = l + N;
  if (p.front) {
    lmoe::GemmArgs a;
    a.A = x; a.lda = d; a.B = w->w_down; a.B2 = w->w_router; a.N0 = static_cast<int>(l);
    a.ldb = d; a.ldc = front_ld;
    a.M = Ti; a.N = static_cast<int>(front_ld); a.K = d;
    LMOE_TRY(lmoe::launch_gemm_tiled(a, adt, lmoe::Dt::F32, p.front_plan.tile, s,
                                     p.front_plan.splits, partial, false),
             "W_down + router GEMM");
  } else if (c.has_projections) {
    lmoe::GemmArgs a;
    a.A = x; a.lda = d; a.B = w->w_down; a.ldb = d; a.C = u; a.ldc = l;
    a.M = Ti; a.N = l; a.K = d;
    if (p.down_grouped) {
      a.a_nrows = Ti; a.max_rows = Ti;
      // grouped experts: the blocked copy of u that FC1 gathers from, stored
      // beside u by the same launch
      if (p.grouped) a.C2 = ws + p.ublk;
      LMOE_TRY(lmoe::launch_gemm_grouped(a, s), "W_down GEMM (grouped)");
    } else {
      LMOE_TRY(lmoe::launch_gemm_tiled(a, adt, adt, p.down.tile, s, p.down.splits, partial,
                                       !p.defer_u),
               "W_down GEMM");
    }
  }
  if (!p.front) {
    const bool lat = c.router_input == LMOE_ROUTER_ON_LATENT;
    lmoe::GemmArgs a;
    a.A = lat ? u : x; a.lda = lat ? l : d;
    a.B = w->w_router; a.ldb = lat ? l : d;
    a.C = logits; a.ldc = N;
    a.M = Ti; a.N = N; a.K = lat ? l : d;
    LMOE_TRY(lmoe::launch_gemm_tiled(a, adt, lmoe::Dt::F32, p.router.tile, s, p.router.splits, part_z,
                                     !p.defer_z),
             "router GEMM");
  }
  LMOE_MARK(1);
  // ---- stage 1: top-k and gates (and the deferred split-K reductions)
  {
    lmoe::TopkArgs a;
    a.logits = p.front ? partial + l : p.defer_z ? part_z : logits;
    a.logits_ld = p.front ? front_ld : N;
    a.logits_sstride = int64_t(Ti) * a.logits_ld;
    a.lsplits = p.front ? p.front_plan.splits : p.defer_z ? p.router.splits : 1;
    a.logits_out = p.defer_z && dbg && dbg->logits ? logits : nullptr;
    a.bias = c.has_router_bias ? w->router_bias : nullptr;
    a.T = Ti; a.N = N; a.K = K; a.gating = c.gating;
    a.idx = idx; a.gate = gate;
    if (p.defer_u) {
      a.u_part = partial;
      a.u_ld = p.front ? front_ld : l;
      a.u_sstride = int64_t(Ti) * a.u_ld;
      a.usplits = p.front ? p.front_plan.splits : p.down.splits;
      a.l = static_cast<int>(l);
      a.u = u; a.u_bf16 = adt == lmoe::Dt::BF16;
    }
    LMOE_TRY(lmoe::launch_topk_gate(a, s), "top-k");
  }
  LMOE_MARK(2);
  // ---- stage 2: dispatch indices
  if (lmoe::route_small_fits(Ti, N, K)) {
    LMOE_TRY(lmoe::launch_route_small(idx, Ti, N, K, route_tile, counts, offsets, tiles, slot_of,
                                      token_of, s, active),
             "route (single workgroup)");
  } else {
    LMOE_TRY(lmoe::launch_route_masks(idx, Ti, N, K, masks, s), "route masks");
    LMOE_TRY(lmoe::launch_route_scan(masks, p.nblk, N, route_tile, counts, offsets, base, tiles, s,
                                     active),
             "route scan");
    LMOE_TRY(lmoe::launch_route_assign(idx, masks, base, offsets, Ti, N, K, slot_of, token_of, s),
             "route assign");
  }
  LMOE_MARK(3);
  // ---- stage 3: FC1 + squared ReLU, token rows gathered through token_of
  // (fused: FC1 and FC2 of each expert in one kernel, H kept on chip)
  if (p.fused) {
    lmoe::FfnArgs a;
    a.A = u; a.lda = l; a.a_rows = token_of; a.a_nrows = Ti;
    a.W1 = w->w1; a.W2 = w->w2;
    a.Y = Y; a.ldy = l;
    a.g_off = offsets; a.G = N;
    a.l = static_cast<int>(l); a.m = static_cast<int>(m);
    a.act = act1;
    if (edt == lmoe::Dt::MXFP4) { a.W1_mx = w->w1_mx; a.W2_mx = w->w2_mx; }
    LMOE_TRY(lmoe::launch_ffn_stream(a, s), "FC1 + FC2 (fused)");
  } else {
    lmoe::GemmArgs a;
    a.A = u; a.lda = l; a.a_rows = token_of; a.a_nrows = Ti;
    const int n1 = glu ? 2 * m : m;  // W1 rows
    a.B = w->w1; a.ldb = l; a.b_gstride = int64_t(n1) * l;
    a.b_scale = edt == lmoe::Dt::FP8 ? w->w1_scale : nullptr; a.s_gstride = n1;
    if (edt == lmoe::Dt::MXFP4) {  // E2M1 pairs: byte strides; a scale per 32
      a.ldb = l / 2; a.b_gstride = int64_t(n1) * (l / 2);
      a.b_mx = w->w1_mx; a.mx_ld = l / 32; a.mx_gstride = int64_t(n1) * (l / 32);
    }
    a.C = H; a.ldc = m;
    a.N = n1; a.K = l;
    a.g_off = offsets; a.g_tiles = tiles; a.G = N; a.max_rows = static_cast<int>(p.copies);
    a.g_active = active;
    a.act = act1;
    if (p.stream) LMOE_TRY(lmoe::launch_gemm_stream(a, adt, edt, adt, p.mb_max, s), "FC1 (stream)");
    else if (edt == lmoe::Dt::FP8) {
      if (w->experts_packed) { a.B = w->experts_packed; a.b_bands = 1; }
      LMOE_TRY(lmoe::launch_gemm_fp8w(a, s), "FC1 (grouped, fp8)");
    }
    else if (p.grouped) {
      // u in 32-column blocks over its T rows: the rows FC1 gathers for an
      // expert are mostly consecutive tokens, whose K-stage pieces then sit
      // side by side
      // (written by the W_down launch when it runs on the grouped kernel)
      void* ub = ws + p.ublk;
      if (!p.down_grouped)
        LMOE_TRY(lmoe::launch_pack_bands(u, ub, 1, Ti, l * ab, Ti, s), "u in blocks");
      a.A = ub; a.a_kblock = Ti;
      // H in 32-column blocks, so that FC2 loads each K stage of its rows as
      // one contiguous block; W1 in 256-row bands when a packed copy is given
      a.c_kblock = static_cast<int>(p.copies);
      if (w->experts_packed) { a.B = w->experts_packed; a.b_bands = 1; }
      LMOE_TRY(lmoe::launch_gemm_grouped(a, s), "FC1 (grouped)");
    }
    else LMOE_TRY(lmoe::launch_gemm_tiled(a, adt, adt, p.expert_tile, s), "FC1 (tiled)");
  }
  LMOE_MARK(4);
  // ---- stage 4: FC2
  if (!p.fused) {
    lmoe::GemmArgs a;
    a.A = H; a.lda = m; a.a_nrows = static_cast<int>(p.copies);
    a.B = w->w2; a.ldb = m; a.b_gstride = int64_t(l) * m;
    a.b_scale = edt == lmoe::Dt::FP8 ? w->w2_scale : nullptr; a.s_gstride = l;
    if (edt == lmoe::Dt::MXFP4) {
      a.ldb = m / 2; a.b_gstride = int64_t(l) * (m / 2);
      a.b_mx = w->w2_mx; a.mx_ld = m / 32; a.mx_gstride = int64_t(l) * (m / 32);
    }
    a.C = Y; a.ldc = l;
    a.N = l; a.K = m;
    a.g_off = offsets; a.g_tiles = tiles; a.G = N; a.max_rows = static_cast<int>(p.copies);
    a.g_active = active;
    a.act = lmoe::kActNone;
    if (p.stream) LMOE_TRY(lmoe::launch_gemm_stream(a, adt, edt, adt, p.mb_max, s), "FC2 (stream)");
    else if (edt == lmoe::Dt::FP8) {
      if (w->experts_packed) {
        const int n1 = glu ? 2 * m : m;
        a.B = static_cast<const char*>(w->experts_packed) + size_t(N) * n1 * l;
        a.b_bands = 1;
      }
      LMOE_TRY(lmoe::launch_gemm_fp8w(a, s), "FC2 (grouped, fp8)");
    }
    else if (p.grouped) {
      a.a_kblock = static_cast<int>(p.copies);   // H as FC1 wrote it
      if (w->experts_packed) {                   // W2 follows W1 in the packed copy
        const int n1 = glu ? 2 * m : m;
        a.B = static_cast<const char*>(w->experts_packed) + size_t(N) * n1 * l * 2;
        a.b_bands = 1;
      }
      LMOE_TRY(lmoe::launch_gemm_grouped(a, s), "FC2 (grouped)");
    }
    else LMOE_TRY(lmoe::launch_gemm_tiled(a, adt, adt, p.expert_tile, s), "FC2 (tiled)");
  }
  LMOE_MARK(5);
  // ---- stage 5: gate-weighted combine (into out directly for the standard
  // MoE, adding the shared experts' R there)
  if (!c.has_projections) LMOE_TRY(join(), "hipStreamWaitEvent (join)");
  LMOE_TRY(lmoe::launch_combine(Y, slot_of, gate, Ti, K, l, adt, c.has_projections ? nullptr : R,
                                v, s),
           "combine");
  LMOE_MARK(6);
  // ---- stage 6: up-projection, + R in its epilogue
  if (c.has_projections) {
    LMOE_TRY(join(), "hipStreamWaitEvent (join)");
    lmoe::GemmArgs a;
    a.A = v; a.lda = l; a.B = w->w_up; a.ldb = l; a.C = out; a.ldc = d;
    a.M = Ti; a.N = d; a.K = l;
    a.R = R; a.ldr = d;
    if (p.up_grouped) {
      a.a_nrows = Ti; a.max_rows = Ti;
      LMOE_TRY(lmoe::launch_gemm_grouped(a, s), "W_up GEMM (grouped)");
    } else {
      LMOE_TRY(lmoe::launch_gemm_tiled(a, adt, adt, p.up.tile, s, p.up.splits, partial), "W_up GEMM");
    }
  }
  LMOE_MARK(7);

  // ---- optional copies of intermediate results
  if (dbg) {
    auto cp = [&](void* dst, const void* src, size_t bytes, const char* what) -> lmoe_status {
      if (!dst || bytes == 0) return LMOE_OK;
      hipError_t r = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
      return r == hipSuccess ? LMOE_OK : hip_fail(r, what);
    };
    lmoe_status st;
    if ((st = cp(dbg->topk_idx, idx, size_t(p.copies) * 4, "copy topk_idx")) != LMOE_OK) return st;
    if ((st = cp(dbg->topk_gate, gate, size_t(p.copies) * 4, "copy topk_gate")) != LMOE_OK) return st;
    if ((st = cp(dbg->expert_counts, counts, size_t(N) * 4, "copy counts")) != LMOE_OK) return st;
    if ((st = cp(dbg->expert_offsets, offsets, size_t(N + 1) * 4, "copy offsets")) != LMOE_OK) return st;
    if ((st = cp(dbg->slot_of, slot_of, size_t(p.copies) * 4, "copy slot_of")) != LMOE_OK) return st;
    if ((st = cp(dbg->token_of, token_of, size_t(p.copies) * 4, "copy token_of")) != LMOE_OK) return st;
    if ((st = cp(dbg->logits, logits, size_t(T) * N * 4, "copy logits")) != LMOE_OK) return st;
    if (c.has_projections &&
        (st = cp(dbg->latent, u, size_t(T) * l * ab, "copy latent")) != LMOE_OK) return st;
  }
#undef LMOE_MARK
#undef LMOE_BEGIN
#undef LMOE_END
#undef LMOE_TRY
  return LMOE_OK;
}

}  // extern "C"

extern "C" {

lmoe_status latentmoe_forward_static(const lmoe_handle* h, const lmoe_weights* w, const void* x,
                                     int64_t T, void* out, const lmoe_debug_out* dbg,
                                     void* stream) {
  if (!h || !w) return fail(LMOE_ERR_INVALID_ARG, "forward_static: NULL handle or weights");
  if (T < 0) return fail(LMOE_ERR_INVALID_ARG, "forward_static: T < 0");
  if (T == 0) return LMOE_OK;
  if (T * h->cfg.top_k > kMaxCopies)
    return fail(LMOE_ERR_UNSUPPORTED, "forward_static: T*K too large");
  const size_t need = make_plan(h->cfg, T).total;
  if (need > size_t(LMOE_STATIC_SCRATCH_BYTES))
    return fail(LMOE_ERR_WORKSPACE,
                "forward_static: %lld tokens need %zu bytes of scratch, more than the %zu the "
                "library holds per device; use latentmoe_forward with a workspace",
                (long long)T, need, size_t(LMOE_STATIC_SCRATCH_BYTES));
  // the device of the call: the stream's, which must be the current one
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "forward_static: hipGetDevice");
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return hip_fail(e, "forward_static: hipStreamGetDevice");
    if (sdev != dev)
      return fail(LMOE_ERR_INVALID_ARG, "forward_static: the stream belongs to device %d, "
                  "the current device is %d", sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LMOE_ERR_UNSUPPORTED, "forward_static: device %d beyond %d", dev, kMaxDevices);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "forward_static: hipGetSymbolAddress(scratch)");
      if (!p) return fail(LMOE_ERR_HIP, "forward_static: no device address for the scratch");
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return latentmoe_forward_overlap(h, w, x, T, out, dbg, ws, size_t(LMOE_STATIC_SCRATCH_BYTES),
                                   stream, nullptr);
}

}  // extern "C"
