/*
 * latentmoe.h -- C ABI of the MI355X (gfx950) LatentMoE layer forward.
 *
 * The operation (LatentMoE: Toward Optimal Accuracy per FLOP and Parameter
 * in Mixture of Experts, §3, Eq. (1) and Eq. (2)):
 *
 *   u   = W_down . x                    latent token, W_down in R^{l x d}
 *   z   = W_r . x   (or W_r . u) [+ b]  router logits over N experts, fp32
 *   T   = K experts with the largest z  ties go to the lower expert id
 *   v   = sum_{i in T} g_i E_i(u; l)    E_i(u) = W2_i . (max(0, W1_i . u))^2,
 *                                       W1_i in R^{m x l}, W2_i in R^{l x m}
 *                                       (SwiGLU experts, §3's W_FC1, W_gate, W_FC2:
 *                                       E_i(u) = W2_i . ((W1_i . u) * SiLU(Wg_i . u)))
 *   out = W_up . v + sum_{j < S} E_j(x; d)       W_up in R^{d x l}
 *
 * The S shared experts (the second sum of Eq. (1)/(2)) run on x in the d
 * space, ungated, with the routed experts' nonlinearity:
 * E_j(x; d) = Ws2_j . (max(0, Ws1_j . x))^2, Ws1_j in R^{m_shared x d},
 * Ws2_j in R^{d x m_shared}.  S = 0 leaves them out.
 *
 * With has_projections == 0 the layer is the standard MoE (l == d, u = x,
 * out = v + shared): the same code path with the two projections skipped.
 *
 * Conventions
 *  - Every tensor is row-major "[out][in]" (y = W . x), dense, with the
 *    shapes given on each field.  All data pointers are DEVICE pointers owned
 *    by the caller; they must be 16-byte aligned.  bf16 values are raw
 *    IEEE bfloat16 bit patterns (uint16), fp8 values raw OCP E4M3 bytes,
 *    MXFP4 values packed E2M1 pairs with E8M0 block-scale bytes.
 *  - The library owns only the handle (host memory).  A handle is immutable
 *    after latentmoe_create and may be shared by concurrent forward calls on
 *    different streams if each call has its own workspace and outputs.
 *  - latentmoe_forward is asynchronous and stream-ordered: it enqueues
 *    kernels on `stream` (a hipStream_t passed as void*, NULL = the null
 *    stream) and returns; it never synchronises the host, never allocates
 *    device memory and never copies data to the host.
 *    latentmoe_forward_overlap may also use a second stream for the shared
 *    experts; the call's outputs are still ordered on `stream`.
 *  - Errors are returned as lmoe_status, never thrown; on a non-OK status
 *    nothing has been enqueued except for LMOE_ERR_HIP (a launch failed
 *    part-way; the stream's outputs are then undefined).
 *    latentmoe_last_error() gives a message for the calling thread.
 */
#ifndef LATENTMOE_H
#define LATENTMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMOE_OK = 0,
  LMOE_ERR_INVALID_ARG = -1,  /* NULL pointer, bad shape, k > N, T < 0, ... */
  LMOE_ERR_UNSUPPORTED = -2,  /* valid in principle but not implemented (e.g. fp8 activations) */
  LMOE_ERR_WORKSPACE = -3,    /* workspace NULL or smaller than latentmoe_workspace_size() */
  LMOE_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
  LMOE_ERR_ALLOC = -5         /* host allocation of the handle failed */
} lmoe_status;

typedef enum {
  LMOE_F32 = 0,
  LMOE_BF16 = 1,
  LMOE_FP8_E4M3_ROWSCALE = 2, /* OCP E4M3 bytes + one fp32 scale per matrix row: w = q * s */
  LMOE_MXFP4_E2M1 = 3         /* OCP MX FP4: E2M1 elements, two per byte (element 2j in the low
                                 nibble of byte j), + one E8M0 scale byte 2^(e-127) per 32
                                 consecutive elements of a row (byte 0 is 2^-127, byte 0xFF
                                 is NaN and makes the block NaN); expert weights only, bf16
                                 activations, l and m multiples of 32, streaming or fused
                                 kernel */
} lmoe_dtype;

typedef enum {
  LMOE_ROUTER_ON_X = 0,       /* z = W_r . x, W_r in R^{N x d}  (§3, text after Eq. (1)) */
  LMOE_ROUTER_ON_LATENT = 1   /* z = W_r . u, W_r in R^{N x l}  (routing "in the latent") */
} lmoe_router_input;

typedef enum {
  LMOE_GATE_SOFTMAX_ALL = 0,      /* p = Softmax(z) over all N; g_i = p_i, no renormalisation (Eq. (1)) */
  LMOE_GATE_SOFTMAX_TOPK = 1,     /* softmax over the K selected logits */
  LMOE_GATE_SIGMOID_TOPK_NORM = 2 /* g_i = sigmoid(z_i) / sum_{j in T} sigmoid(z_j) */
} lmoe_gating;

typedef enum {
  LMOE_ACT_SQRELU = 0,            /* non-gated expert FFN with (max(0, a))^2 (Table 2: Squared-ReLU) */
  LMOE_ACT_SWIGLU = 1             /* gated: (W_FC1 . u) * SiLU(W_gate . u), SiLU(b) = b / (1 + e^-b)
                                     (§3's expert matrices; Table 2: SwiGLU).  The FC1 and gate
                                     matrices are passed interleaved by rows, see lmoe_weights */
} lmoe_activation;

/* Expert-FFN kernels (the grouped latent expert FFN of Eq. (2)).  AUTO picks
 * from the mean number of token copies per expert, T*K/N:
 *   STREAM - weight-streaming grouped GEMMs, FC1 then FC2 (few rows per
 *            expert: the decode regime, bound by reading the expert weights);
 *   FUSED  - FC1 and FC2 in one kernel, the activated rows kept on chip
 *            (decode regime, bf16 tokens, bf16 or MXFP4 experts, m <= 1536,
 *            at least one expert per compute unit; an expert with more than
 *            48 rows takes several passes);
 *   TILED  - LDS-tiled MFMA grouped GEMMs (many rows per expert: prefill).
 * Every choice computes the same function; forcing one is for tests and
 * measurements.  FUSED needs bf16 activations, bf16 or MXFP4 experts,
 * m <= 1536, and each expert weight array (all N experts) below 2 GiB;
 * MXFP4 experts never run TILED (AUTO streams them, or runs FUSED). */
typedef enum {
  LMOE_EXPERTS_AUTO = 0,
  LMOE_EXPERTS_TILED = 1,
  LMOE_EXPERTS_STREAM = 2,
  LMOE_EXPERTS_FUSED = 3
} lmoe_expert_kernel;

typedef struct {
  int64_t d;           /* model width */
  int64_t l;           /* latent width (== d when has_projections == 0) */
  int64_t m;           /* expert FFN width */
  int64_t n_experts;   /* N, 1 .. 2048 */
  int64_t top_k;       /* K, 1 .. min(N, 64) */
  int32_t router_input;   /* lmoe_router_input */
  int32_t gating;         /* lmoe_gating */
  int32_t activation;     /* lmoe_activation */
  int32_t act_dtype;      /* LMOE_F32 | LMOE_BF16: x, W_down, W_router, W_up, out */
  int32_t expert_dtype;   /* LMOE_F32 | LMOE_BF16 | LMOE_FP8_E4M3_ROWSCALE | LMOE_MXFP4_E2M1:
                             W1, W2.  F32 experts need F32 activations; the others BF16. */
  int32_t has_projections;  /* 0: standard MoE (requires l == d) */
  int32_t has_router_bias;  /* 1: z += b before selection and gating (fp32 b[N]) */
  int32_t expert_kernel;    /* lmoe_expert_kernel; 0 = AUTO */
  int64_t n_shared;         /* S shared experts, 0 .. 64 (Eq. (1)/(2), second sum) */
  int64_t m_shared;         /* their FFN width, a multiple of 16 (read when n_shared > 0) */
} lmoe_config;

/* Device pointers; shapes use the config's d, l, m, N.  With SwiGLU experts
 * (activation LMOE_ACT_SWIGLU) the up-projection and gate matrices travel
 * as one interleaved matrix: w1 is [N][2m][l] with row 2i = W_FC1 row i and
 * row 2i + 1 = W_gate row i of the expert (w1_scale [N][2m] and w1_mx
 * [N][2m][l/32] likewise), and
 * w_shared1 is [2*S*m_shared][d] with row 2k = Ws_FC1 row k and row 2k + 1 =
 * Ws_gate row k (expert j's rows start at 2*j*m_shared). */
typedef struct {
  const void *w_down;       /* [l][d] act dtype; NULL without projections */
  const void *w_router;     /* [N][d] (ROUTER_ON_X) or [N][l] (ROUTER_ON_LATENT), act dtype */
  const float *router_bias; /* [N] fp32; only read when has_router_bias */
  const void *w1;           /* [N][m][l] expert dtype ([N][2m][l] interleaved with SwiGLU;
                               MXFP4: bytes [N][m][l/2], or [N][2m][l/2]) */
  const void *w2;           /* [N][l][m] expert dtype (MXFP4: bytes [N][l][m/2]) */
  const float *w1_scale;    /* [N][m] fp32 ([N][2m] with SwiGLU); FP8 experts only */
  const float *w2_scale;    /* [N][l] fp32; FP8 experts only */
  const void *w_up;         /* [d][l] act dtype; NULL without projections */
  const void *w_shared1;    /* [S*m_shared][d] act dtype: Ws1_j is rows j*m_shared ..; n_shared > 0 */
  const void *w_shared2;    /* [d][S*m_shared] act dtype: Ws2_j is columns j*m_shared ..; n_shared > 0 */
  const uint8_t *w1_mx;     /* MXFP4 experts: E8M0 scales [N][m][l/32] of w1 ([N][m][l/2] bytes) */
  const uint8_t *w2_mx;     /* MXFP4 experts: E8M0 scales [N][l][m/32] of w2 ([N][l][m/2] bytes) */
  const void *experts_packed; /* optional: w1 and w2 as latentmoe_pack_expert_weights wrote
                                 them; read by the grouped bf16 and fp8 kernels, NULL = w1, w2 */
} lmoe_weights;

/* Per-stage GPU timing: an opaque object holding HIP events.  Attach one to
 * a forward call through lmoe_debug_out.timer; the call then records an
 * event at the beginning and at the end of each stage (the shared-expert
 * stage on the stream it runs on).  Reading synchronises on those events and
 * ADDS the stage durations to the accumulators.  With the shared experts on
 * a side stream, the stage that adds their sum (UP, or COMBINE for the
 * standard MoE) includes any wait for them. */
typedef struct lmoe_timer lmoe_timer;

enum {
  LMOE_STAGE_DOWN_ROUTER = 0, /* W_down GEMM and router-logit GEMM */
  LMOE_STAGE_TOPK = 1,        /* top-k + gating */
  LMOE_STAGE_DISPATCH = 2,    /* expert histogram, prefix sum, stable slot assignment */
  LMOE_STAGE_FC1 = 3,         /* grouped latent FC1 + squared ReLU or SwiGLU (gathers u rows);
                                 the fused kernel runs FC1 and FC2 here */
  LMOE_STAGE_FC2 = 4,         /* grouped latent FC2 */
  LMOE_STAGE_COMBINE = 5,     /* gate-weighted sum of the K expert outputs per token */
  LMOE_STAGE_UP = 6,          /* W_up GEMM (+ the shared experts' sum) */
  LMOE_STAGE_SHARED = 7,      /* shared experts: x Ws1^T + activation, then . Ws2^T (fp32) */
  LMOE_NUM_STAGES = 8
};

/* Optional device outputs of a forward call (any may be NULL). */
typedef struct {
  int32_t *topk_idx;       /* [T][K] selected expert ids, by (z desc, id asc) */
  float *topk_gate;        /* [T][K] gate of topk_idx[t][j] */
  int32_t *expert_counts;  /* [N] copies routed to each expert; sums to T*K */
  int32_t *expert_offsets; /* [N+1] exclusive prefix sum of expert_counts */
  int32_t *slot_of;        /* [T][K] row of copy (t, j) in the expert-grouped order */
  int32_t *token_of;       /* [T*K] token of each expert-grouped row; within an
                              expert, rows follow increasing token index */
  float *logits;           /* [T][N] fp32 router logits W_r . x (or . u), before the bias */
  void *latent;            /* [T][l] u in act dtype (projections only) */
  lmoe_timer *timer;       /* host object from latentmoe_timer_create, or NULL */
} lmoe_debug_out;

typedef struct lmoe_handle lmoe_handle;

/* Validate `cfg` and build a handle (host only; no HIP call).
 * Returns INVALID_ARG for inconsistent shapes (k > N, l != d without
 * projections, non-positive sizes), UNSUPPORTED for combinations this
 * build does not implement (d, l, m not multiples of 16; N > 2048;
 * K > 64; activation/expert dtype pairs other than f32/f32, bf16/bf16,
 * bf16/fp8 and bf16/MXFP4; MXFP4 with l or m not multiples of 32 or with a
 * forced tiled or fused expert kernel). */
lmoe_status latentmoe_create(const lmoe_config *cfg, lmoe_handle **out);

/* Bytes of device workspace a forward call over T tokens needs. */
lmoe_status latentmoe_workspace_size(const lmoe_handle *h, int64_t T, size_t *bytes);

/* Expert weights in a second layout, for the grouped expert GEMMs of large
 * batches: each expert matrix is stored in bands of rows, a band as its
 * 64-byte column blocks one after another, a block as the band's rows of
 * 64 bytes each.  bf16 experts (prefill; W1's and W2's row counts multiples
 * of 256, l and m of 32): 256-row bands, so that a K stage of a 256-row
 * weight tile is one contiguous 16 KB block instead of 256 row pieces.
 * fp8 experts (l and m multiples of 64): 16-row bands, the rows that one
 * wave of the fp8 kernel streams, so that each of its loads reads 1 KB in
 * one piece.  The row scales stay where they are.  The expert FFN of
 * Eq. (2) is unchanged: results are bit-identical with and without the
 * packed copy.
 *
 * latentmoe_packed_weights_size: bytes of the packed copy (W1 then W2, as
 * large as the two matrices), or 0 when the layer's experts have no packed
 * form (f32 or MXFP4 experts, or shapes the kernels above do not take).
 *
 * latentmoe_pack_expert_weights: writes the packed copy of w->w1 and w->w2
 * into `packed` (device memory owned by the caller, >= the size above,
 * 16-byte aligned, not overlapping them), enqueued on `stream`.  Pass it
 * as lmoe_weights.experts_packed to forward calls, together with w1 and w2
 * (the other expert kernels read those: the packed copy is read where a
 * batch runs the grouped bf16 or the fp8 tiled expert kernel, see
 * latentmoe_expert_regime); keep it in step with w1 and w2.
 * Returns UNSUPPORTED when the size is 0, WORKSPACE when packed_bytes is
 * too small, INVALID_ARG for NULL or misaligned pointers, HIP on a launch
 * error. */
size_t latentmoe_packed_weights_size(const lmoe_handle *h);
lmoe_status latentmoe_pack_expert_weights(const lmoe_handle *h, const lmoe_weights *w, void *packed,
                                          size_t packed_bytes, void *stream);

/* out[T][d] (act dtype) = layer(x[T][d]).  T == 0 is a no-op returning OK.
 * `workspace` (device, >= latentmoe_workspace_size bytes, 256-byte aligned)
 * is scratch owned by the caller for the duration of the call on `stream`.
 * `dbg` may be NULL. */
lmoe_status latentmoe_forward(const lmoe_handle *h, const lmoe_weights *w, const void *x,
                              int64_t T, void *out, const lmoe_debug_out *dbg,
                              void *workspace, size_t workspace_bytes, void *stream);

/* A second stream for the shared experts (LatentMoE §4.3 names separate
 * streams for routed and shared experts as a way to cut latency when the
 * routed path leaves the GPU partly idle).  The object holds the side
 * stream (a hipStream_t as void*, owned by the caller, on the device of the
 * forward calls, not NULL, default priority) and two events of its own.
 * One forward call at a time may use an lmoe_overlap. */
typedef struct lmoe_overlap lmoe_overlap;
lmoe_status latentmoe_overlap_create(void *side_stream, lmoe_overlap **out);
lmoe_status latentmoe_overlap_destroy(lmoe_overlap *o);

/* latentmoe_forward with the shared experts on ov's side stream: forked
 * from `stream` at the start of the call (they read only x) and joined back
 * before the stage that adds their sum.  ov == NULL (or n_shared == 0) is
 * latentmoe_forward.  The side stream must differ from `stream`. */
lmoe_status latentmoe_forward_overlap(const lmoe_handle *h, const lmoe_weights *w, const void *x,
                                      int64_t T, void *out, const lmoe_debug_out *dbg,
                                      void *workspace, size_t workspace_bytes, void *stream,
                                      lmoe_overlap *ov);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * latentmoe_forward with the workspace taken from a scratch array the
 * library holds in device memory, LMOE_STATIC_SCRATCH_BYTES per device (each
 * GPU the library runs on holds its copy until the process ends).  The call
 * allocates nothing; the caller still passes x, out and the weights.  The
 * shared experts run on `stream` (no side stream).  `stream` must belong to
 * the current device (NULL = its null stream).  Returns LMOE_ERR_WORKSPACE,
 * enqueuing nothing, when latentmoe_workspace_size(T) exceeds
 * LMOE_STATIC_SCRATCH_BYTES (64 MiB: the decode layers up to T = 512 fit,
 * e.g. d 4096, l 1024, m 1536, N 512, K 32; the prefill batches do not).
 * Every call on one device shares that device's scratch and leaves the last
 * call's contents in it (nothing in it needs to start at zero): calls that
 * overlap on one device -- on two streams, or from two threads without
 * stream order -- race on it and give undefined results. */
#define LMOE_STATIC_SCRATCH_BYTES (64u << 20)
lmoe_status latentmoe_forward_static(const lmoe_handle *h, const lmoe_weights *w, const void *x,
                                     int64_t T, void *out, const lmoe_debug_out *dbg,
                                     void *stream);

lmoe_status latentmoe_destroy(lmoe_handle *h);

/* Stage timer: create/destroy, and read the accumulated milliseconds per
 * stage (LMOE_NUM_STAGES floats) and the number of recorded forward calls.
 * Reading waits for the last recorded forward call to finish and resets. */
lmoe_status latentmoe_timer_create(lmoe_timer **out);
lmoe_status latentmoe_timer_read(lmoe_timer *t, float *stage_ms, int32_t n_stages,
                                 int32_t *n_calls);
lmoe_status latentmoe_timer_destroy(lmoe_timer *t);

/* Static strings; never NULL. */
const char *latentmoe_status_string(lmoe_status s);
const char *latentmoe_last_error(void);

/* Name of the expert-kernel regime the handle picks for T tokens:
 * "stream" (weight-streaming grouped GEMMs, tokens per expert few),
 * "fused" (FC1 and FC2 in one weight-streaming kernel), "tiled"
 * (LDS-tiled MFMA grouped GEMMs), "grouped" (the persistent 256 x 256
 * MFMA grouped GEMMs of bf16 layers with many tokens per expert) or "fp8w"
 * (the grouped GEMMs over fp8 weights streamed into registers, which the
 * TILED choice selects for fp8 experts).  For reports only. */
const char *latentmoe_expert_regime(const lmoe_handle *h, int64_t T);

#ifdef __cplusplus
}
#endif
#endif /* LATENTMOE_H */
