/*
 * latentmoe_oracle.h -- plain, slow, fp64 CPU oracle of one LatentMoE layer
 * forward.  TEST INFRASTRUCTURE ONLY: it exists to check the GPU library.
 * Only the test suite, the package smoke check and the benchmark's CPU
 * baseline leg may load it; the GPU library never includes, links or calls
 * it, and it shares no source with the GPU library.
 *
 * What it computes (LatentMoE: Toward Optimal Accuracy per FLOP and
 * Parameter in Mixture of Experts, §3, Eq. (1) and Eq. (2)):
 *
 *   u      = W_down . x                     (u = x for the standard MoE)
 *   z      = W_r . x  (or W_r . u)  [+ b]   router logits
 *   T      = indices of the K largest z     (ties: lower expert id first)
 *   g_i    = gate of expert i in T           (three gating rules, below)
 *   v      = sum_{i in T, ascending i} g_i * W2_i . f(W1_i . u, Wg_i . u)
 *   out    = W_up . v                        (out = v for the standard MoE)
 *            + sum_{j < S} Ws2_j . f(Ws1_j . x, Wsg_j . x)   shared experts
 *
 * Expert nonlinearity f (§3 parameterises an expert by W_FC1, W_gate and
 * W_FC2; Table 2 names SwiGLU and Squared-ReLU): activation 0, the
 * Squared-ReLU FFN, f(a, .) = (max(0, a))^2 with no gate matrix; activation
 * 1, SwiGLU, f(a, b) = a * SiLU(b) = a * b / (1 + exp(-b)), b the gate.
 *
 * The S shared experts run on x in the d space, ungated (the second sum of
 * Eq. (1)/(2)); their nonlinearity is the routed experts' Squared-ReLU FFN
 * and their hidden width m_shared is a free parameter (the paper gives no
 * separate width for them).  S = 0 drops the term.
 *
 * Gating rules: 0 = softmax over all N logits, gate = p_i of the selected
 * experts with no renormalisation (Eq. (1)); 1 = softmax over the K selected
 * logits; 2 = sigmoid of the selected logits normalised to sum to one.
 * Every sum runs in ascending index order, in fp64, with no intermediate
 * rounding; stored bf16, fp8 and MXFP4 values are upcast exactly (fp8 as
 * q * row scale, MXFP4 as e2m1 * 2^(e8m0 - 127)).
 * The router reads the unrounded fp64 x or u, like every other step.
 */
#ifndef LATENTMOE_ORACLE_H
#define LATENTMOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3_ROWSCALE = 2, ORC_MXFP4 = 3 };
enum { ORC_SOFTMAX_ALL = 0, ORC_SOFTMAX_TOPK = 1, ORC_SIGMOID_TOPK_NORM = 2 };
enum { ORC_SQRELU = 0, ORC_SWIGLU = 1 };

typedef struct {
  int64_t d, l, m, n_experts, top_k;
  int32_t router_on_latent;  /* 0: router reads x (d wide); 1: reads u (l wide) */
  int32_t gating;            /* ORC_SOFTMAX_ALL | ORC_SOFTMAX_TOPK | ORC_SIGMOID_TOPK_NORM */
  int32_t has_projections;   /* 0: standard MoE, requires l == d */
  int32_t has_router_bias;
  int32_t act_dtype;         /* ORC_F32 | ORC_BF16: x, W_down, W_router, W_up */
  int32_t expert_dtype;      /* ORC_F32 | ORC_BF16 | ORC_FP8_E4M3_ROWSCALE | ORC_MXFP4: W1, W2 */
  int64_t n_shared;          /* S >= 0 shared experts */
  int64_t m_shared;          /* their hidden width (> 0 when S > 0) */
  int32_t activation;        /* ORC_SQRELU | ORC_SWIGLU */
} orc_layer;

/* Host pointers, row-major [out][in]: w_down [l][d], w_router [N][d or l],
 * router_bias [N] fp32, w1 [N][m][l], w2 [N][l][m], w1_scale [N][m],
 * w2_scale [N][l] (fp8 only), w_up [d][l]; shared experts in the activation
 * dtype: w_shared1 [S*m_shared][d] (expert j owns rows j*m_shared ..),
 * w_shared2 [d][S*m_shared] (expert j owns columns j*m_shared ..).  SwiGLU
 * only: w_gate [N][m][l] in the expert dtype (+ w_gate_scale [N][m] for
 * fp8), w_shared_gate [S*m_shared][d] in the activation dtype.  MXFP4
 * experts (OCP MX, E2M1 elements, one E8M0 scale per 32 consecutive
 * elements of a row): w1 [N][m][l/2], w2 [N][l][m/2] and w_gate bytes with
 * element 2j in the low nibble of byte j; w1_mx [N][m][l/32], w2_mx
 * [N][l][m/32], w_gate_mx [N][m][l/32] the scales (l, m multiples of 32). */
typedef struct {
  const void *w_down, *w_router;
  const float *router_bias;
  const void *w1, *w2;
  const float *w1_scale, *w2_scale;
  const void *w_up;
  const void *w_shared1, *w_shared2;
  const void *w_gate;
  const float *w_gate_scale;
  const void *w_shared_gate;
  const uint8_t *w1_mx, *w2_mx, *w_gate_mx;
} orc_weights;

/* Sparse forward (the definition).  x holds all tokens ([*][d], act dtype).
 * tok: n token indices to evaluate (NULL = 0..n-1).  forced: optional
 * [n][K] expert ids used instead of the top-K selection (gates are then
 * computed for that set).  Outputs, all [n][...]:
 *   out [n][d]; idx [n][K] int32, ordered by (z desc, id asc);
 *   gate [n][K] (gate of idx[j]); margin [n] = z_(K) - z_(K+1) in fp64
 *   (+inf when K == N); logits [n][N] (nullable); latent [n][l] (nullable).
 * Returns 0, or -1 on invalid arguments.  OpenMP-parallel over tokens. */
int orc_forward(const orc_layer *L, const orc_weights *W, const void *x, const int64_t *tok,
                int64_t n, const int32_t *forced, double *out, int32_t *idx, double *gate,
                double *margin, double *logits, double *latent);

/* Brute-force dense reference: every expert is evaluated for every token,
 * selection is by rank counting (expert e is chosen iff fewer than K
 * experts beat it under (z desc, id asc)), and the expert outputs are
 * mixed with a dense gate row G[n][N] (zero for unchosen experts) summed
 * over all experts in ascending order.  out [n][d], gate_dense [n][N]. */
int orc_forward_dense(const orc_layer *L, const orc_weights *W, const void *x,
                      const int64_t *tok, int64_t n, double *out, double *gate_dense);

/* Routing only (§3: logits, then the top-K set T_{K,N'}), for tokens 0 .. n-1:
 * idx [n][K] ordered by (z desc, id asc), margin [n] = z_(K) - z_(K+1)
 * (+inf when K == N), logits [n][N] (nullable), the same values orc_forward
 * returns for them.  No expert is evaluated.  Returns 0, or -1 on invalid
 * arguments. */
int orc_route(const orc_layer *L, const orc_weights *W, const void *x, int64_t n, int32_t *idx,
              double *margin, double *logits);

/* Exact upcasts of the storage formats. */
double orc_bf16_to_f64(uint16_t bits);
double orc_e4m3_to_f64(uint8_t code); /* OCP E4M3: bias 7, S.1111.111 = NaN */
double orc_e2m1_to_f64(uint8_t code); /* OCP MX FP4 E2M1 (low 4 bits of code) */
double orc_e8m0_to_f64(uint8_t e);    /* OCP MX scale 2^(e-127); 0xFF = NaN */

/* Threads of the OpenMP token loops (the results do not depend on them). */
void orc_set_threads(int n);
int orc_max_threads(void);

/* Per-expert copy counts from an [n][K] id table. */
void orc_expert_counts(const int32_t *idx, int64_t n, int64_t K, int64_t N, int64_t *counts);

#ifdef __cplusplus
}
#endif
#endif
