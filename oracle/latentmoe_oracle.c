/*
 * latentmoe_oracle.c -- fp64 CPU oracle of the LatentMoE layer forward.
 * TEST INFRASTRUCTURE ONLY (see latentmoe_oracle.h): never part of the GPU
 * library, shares no source with it.
 *
 * Follows LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in
 * Mixture of Experts, §3 (matrix shapes of W_down, W_FC1, W_FC2, W_up;
 * routing weights p' = Softmax(W'_r x) from the d-dimensional x; top-K set
 * T_{K,N'}) and Eq. (1)/(2).  The expert nonlinearity is the non-gated
 * Squared-ReLU FFN, W_FC2 . (max(0, W_FC1 . u))^2 (Table 2 lists Squared-ReLU
 * for the 4096-wide models), or the gated SwiGLU FFN over the three matrices
 * §3 gives an expert, W_FC2 . ((W_FC1 . u) * SiLU(W_gate . u)) (Table 2 lists
 * SwiGLU for the 2048-wide model).  The shared experts E_j(x; d) of
 * Eq. (1)/(2) are the same FFN on x in the d space, added to the output
 * ungated.
 */
#define _GNU_SOURCE /* qsort_r */
#include "latentmoe_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

double orc_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign, 4 exponent (bias 7),
 * 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the single
 * pattern with exponent 1111 and mantissa 111 is NaN; no infinities. */
double orc_e4m3_to_f64(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* OCP MX FP4 element, E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit;
 * exponent field 0 is subnormal (m * 0.5); no infinities or NaN.  The eight
 * magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double orc_e2m1_to_f64(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* OCP MX shared scale, E8M0: 2^(e - 127); 0xFF is NaN. */
double orc_e8m0_to_f64(uint8_t e) { return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127); }

/* element i of a tensor stored as `dtype`: fp8 times its row's scale; MXFP4
 * two elements per byte (element 2j in the low nibble of byte j) times the
 * E8M0 scale of its block of 32 (block i / 32: rows hold whole blocks) */
static inline double ld(const void *p, int dtype, int64_t i, const float *scale, int64_t srow,
                        const uint8_t *mx) {
  switch (dtype) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t *)p)[i]);
    case ORC_FP8_E4M3_ROWSCALE:
      return orc_e4m3_to_f64(((const uint8_t *)p)[i]) * (double)scale[srow];
    default: {
      const uint8_t b = ((const uint8_t *)p)[i >> 1];
      return orc_e2m1_to_f64((i & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15)) *
             orc_e8m0_to_f64(mx[i >> 5]);
    }
  }
}

static int check(const orc_layer *L, const orc_weights *W, const void *x, int64_t n) {
  if (!L || !W || !x || n < 0) return -1;
  if (L->d <= 0 || L->l <= 0 || L->m <= 0 || L->n_experts <= 0) return -1;
  if (L->top_k <= 0 || L->top_k > L->n_experts) return -1;
  if (!L->has_projections && L->l != L->d) return -1;
  if (L->has_projections && (!W->w_down || !W->w_up)) return -1;
  if (!W->w_router || !W->w1 || !W->w2) return -1;
  if (L->has_router_bias && !W->router_bias) return -1;
  if (L->expert_dtype == ORC_FP8_E4M3_ROWSCALE && (!W->w1_scale || !W->w2_scale)) return -1;
  if (L->expert_dtype == ORC_MXFP4) {
    if (!W->w1_mx || !W->w2_mx || L->l % 32 || L->m % 32) return -1;
    if (L->activation == ORC_SWIGLU && !W->w_gate_mx) return -1;
  }
  if (L->expert_dtype < ORC_F32 || L->expert_dtype > ORC_MXFP4) return -1;
  if (L->act_dtype != ORC_F32 && L->act_dtype != ORC_BF16) return -1;
  if (L->gating < 0 || L->gating > 2) return -1;
  if (L->n_shared < 0) return -1;
  if (L->n_shared > 0 && (L->m_shared <= 0 || !W->w_shared1 || !W->w_shared2)) return -1;
  if (L->activation != ORC_SQRELU && L->activation != ORC_SWIGLU) return -1;
  if (L->activation == ORC_SWIGLU) {
    if (!W->w_gate) return -1;
    if (L->expert_dtype == ORC_FP8_E4M3_ROWSCALE && !W->w_gate_scale) return -1;
    if (L->n_shared > 0 && !W->w_shared_gate) return -1;
  }
  return 0;
}

/* z = W_r . r [+ b], r = x (d wide) or the latent u (l wide): the router
 * logits over the N experts, from the unrounded fp64 input. */
static void router_logits(const orc_layer *L, const orc_weights *W, const double *xt,
                          const double *u, double *z) {
  const double *rin = L->router_on_latent ? u : xt;
  const int64_t rw = L->router_on_latent ? L->l : L->d;
  for (int64_t e = 0; e < L->n_experts; ++e) {
    double s = 0.0;
    for (int64_t c = 0; c < rw; ++c) s += ld(W->w_router, L->act_dtype, e * rw + c, NULL, 0, NULL) * rin[c];
    if (L->has_router_bias) s += (double)W->router_bias[e];
    z[e] = s;
  }
}

/* Token t's input x_t (d) and latent u_t = W_down . x_t (l; u = x for the
 * standard MoE). */
static void input_and_latent(const orc_layer *L, const orc_weights *W, const void *x, int64_t t,
                             double *xt, double *u) {
  const int64_t d = L->d, l = L->l;
  for (int64_t c = 0; c < d; ++c) xt[c] = ld(x, L->act_dtype, t * d + c, NULL, 0, NULL);
  if (L->has_projections) {
    for (int64_t r = 0; r < l; ++r) {        /* u = W_down . x, W_down in R^{l x d} */
      double s = 0.0;
      for (int64_t c = 0; c < d; ++c) s += ld(W->w_down, L->act_dtype, r * d + c, NULL, 0, NULL) * xt[c];
      u[r] = s;
    }
  } else {
    for (int64_t c = 0; c < d; ++c) u[c] = xt[c];
  }
}

/* Steps shared by the sparse and the dense evaluation of one token:
 * latent u (l) and router logits z (N). */
static void latent_and_logits(const orc_layer *L, const orc_weights *W, const void *x, int64_t t,
                              double *xt, double *u, double *z) {
  input_and_latent(L, W, x, t, xt, u);
  router_logits(L, W, xt, u, z);
}

/* The nonlinearity between the two expert matrices: a = W_FC1 row . input,
 * b = W_gate row . input (SwiGLU only). */
static double act_fn(int activation, double a, double b) {
  if (activation == ORC_SWIGLU) return a * (b / (1.0 + exp(-b)));  /* a * SiLU(b) */
  double r = a > 0.0 ? a : 0.0;
  return r * r;
}

/* y = W2_e . f(W1_e . u, Wg_e . u) : one latent expert E_e(u; l). */
static void expert_ffn(const orc_layer *L, const orc_weights *W, int64_t e, const double *u,
                       double *h, double *y) {
  const int64_t l = L->l, m = L->m;
  const int dt = L->expert_dtype;
  for (int64_t r = 0; r < m; ++r) {
    double s = 0.0, sg = 0.0;
    const int64_t row = e * m + r;
    for (int64_t c = 0; c < l; ++c) s += ld(W->w1, dt, row * l + c, W->w1_scale, row, W->w1_mx) * u[c];
    if (L->activation == ORC_SWIGLU)
      for (int64_t c = 0; c < l; ++c)
        sg += ld(W->w_gate, dt, row * l + c, W->w_gate_scale, row, W->w_gate_mx) * u[c];
    h[r] = act_fn(L->activation, s, sg);
  }
  for (int64_t r = 0; r < l; ++r) {
    double s = 0.0;
    const int64_t row = e * l + r;
    for (int64_t c = 0; c < m; ++c) s += ld(W->w2, dt, row * m + c, W->w2_scale, row, W->w2_mx) * h[c];
    y[r] = s;
  }
}

/* out = W_up . v (or v) */
static void up_project(const orc_layer *L, const orc_weights *W, const double *v, double *out) {
  const int64_t d = L->d, l = L->l;
  if (!L->has_projections) {
    for (int64_t c = 0; c < d; ++c) out[c] = v[c];
    return;
  }
  for (int64_t r = 0; r < d; ++r) {
    double s = 0.0;
    for (int64_t c = 0; c < l; ++c) s += ld(W->w_up, L->act_dtype, r * l + c, NULL, 0, NULL) * v[c];
    out[r] = s;
  }
}

/* out += sum_j E_j(x; d): the S shared experts, evaluated as one
 * concatenated FFN: hs[j*ms + r] = (max(0, Ws1[j*ms + r] . x))^2, then
 * out[r] += sum_k Ws2[r][k] hs[k] over k = 0 .. S*ms-1 in ascending order
 * (expert j's terms are the k in [j*ms, (j+1)*ms)). */
static void add_shared(const orc_layer *L, const orc_weights *W, const double *xt, double *hs,
                       double *out) {
  const int64_t d = L->d, H = L->n_shared * L->m_shared;
  for (int64_t k = 0; k < H; ++k) {
    double s = 0.0, sg = 0.0;
    for (int64_t c = 0; c < d; ++c) s += ld(W->w_shared1, L->act_dtype, k * d + c, NULL, 0, NULL) * xt[c];
    if (L->activation == ORC_SWIGLU)
      for (int64_t c = 0; c < d; ++c)
        sg += ld(W->w_shared_gate, L->act_dtype, k * d + c, NULL, 0, NULL) * xt[c];
    hs[k] = act_fn(L->activation, s, sg);
  }
  for (int64_t r = 0; r < d; ++r) {
    double s = 0.0;
    for (int64_t k = 0; k < H; ++k) s += ld(W->w_shared2, L->act_dtype, r * H + k, NULL, 0, NULL) * hs[k];
    out[r] += s;
  }
}

/* order: (z desc, id asc) */
static int cmp_desc(const void *a, const void *b, void *zv) {
  const double *z = (const double *)zv;
  int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
  if (z[i] > z[j]) return -1;
  if (z[i] < z[j]) return 1;
  return (i > j) - (i < j);
}

static void sort_by_score(int32_t *ord, int64_t N, const double *z) {
  for (int64_t e = 0; e < N; ++e) ord[e] = (int32_t)e;
  qsort_r(ord, (size_t)N, sizeof(int32_t), cmp_desc, (void *)z);
}

/* Gates of the selected set sel[0..K) (ascending ids not required); all
 * sums over expert ids in ascending order. */
static void gates_for(const orc_layer *L, const double *z, const int32_t *sel, int64_t K,
                      double *g) {
  const int64_t N = L->n_experts;
  if (L->gating == ORC_SIGMOID_TOPK_NORM) {
    /* s_i = 1 / (1 + exp(-z_i)); g_i = s_i / sum_{j in T} s_j */
    double tot = 0.0;
    for (int64_t e = 0; e < N; ++e)
      for (int64_t j = 0; j < K; ++j)
        if (sel[j] == e) tot += 1.0 / (1.0 + exp(-z[e]));
    for (int64_t j = 0; j < K; ++j) g[j] = (1.0 / (1.0 + exp(-z[sel[j]]))) / tot;
    return;
  }
  double mx = -INFINITY;
  for (int64_t e = 0; e < N; ++e) if (z[e] > mx) mx = z[e];
  double tot = 0.0;
  if (L->gating == ORC_SOFTMAX_ALL) {
    /* p = Softmax(z) over all N; the selected experts keep p_i as is */
    for (int64_t e = 0; e < N; ++e) tot += exp(z[e] - mx);
  } else {
    /* softmax restricted to the selected logits */
    for (int64_t e = 0; e < N; ++e)
      for (int64_t j = 0; j < K; ++j)
        if (sel[j] == e) tot += exp(z[e] - mx);
  }
  for (int64_t j = 0; j < K; ++j) g[j] = exp(z[sel[j]] - mx) / tot;
}

int orc_forward(const orc_layer *L, const orc_weights *W, const void *x, const int64_t *tok,
                int64_t n, const int32_t *forced, double *out, int32_t *idx, double *gate,
                double *margin, double *logits, double *latent) {
  if (check(L, W, x, n) || !out || !idx || !gate || !margin) return -1;
  const int64_t d = L->d, l = L->l, m = L->m, N = L->n_experts, K = L->top_k;
  int bad = 0;
#pragma omp parallel
  {
    double *xt = malloc(sizeof(double) * (size_t)d);
    double *u = malloc(sizeof(double) * (size_t)(l > d ? l : d));
    double *z = malloc(sizeof(double) * (size_t)N);
    double *h = malloc(sizeof(double) * (size_t)m);
    double *y = malloc(sizeof(double) * (size_t)l);
    double *v = malloc(sizeof(double) * (size_t)l);
    int32_t *ord = malloc(sizeof(int32_t) * (size_t)N);
    int32_t *asc = malloc(sizeof(int32_t) * (size_t)K);
    double *g = malloc(sizeof(double) * (size_t)K);
    double *hs = malloc(sizeof(double) * (size_t)(L->n_shared * L->m_shared + 1));
    const int ok = xt && u && z && h && y && v && ord && asc && g && hs;
    /* every thread reaches the worksharing loop; one without buffers only flags */
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < n; ++i) {
        if (!ok) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        const int64_t t = tok ? tok[i] : i;
        latent_and_logits(L, W, x, t, xt, u, z);
        if (logits) memcpy(logits + i * N, z, sizeof(double) * (size_t)N);
        if (latent) memcpy(latent + i * l, u, sizeof(double) * (size_t)l);
        sort_by_score(ord, N, z);
        margin[i] = K < N ? z[ord[K - 1]] - z[ord[K]] : INFINITY;
        const int32_t *sel = forced ? forced + i * K : ord;
        for (int64_t j = 0; j < K; ++j) idx[i * K + j] = sel[j];
        gates_for(L, z, sel, K, g);
        for (int64_t j = 0; j < K; ++j) gate[i * K + j] = g[j];
        /* experts of the set in ascending id order */
        int64_t na = 0;
        for (int64_t e = 0; e < N; ++e)
          for (int64_t j = 0; j < K; ++j)
            if (sel[j] == e) { asc[na++] = (int32_t)j; break; }
        for (int64_t c = 0; c < l; ++c) v[c] = 0.0;
        for (int64_t a = 0; a < na; ++a) {
          const int64_t j = asc[a];
          expert_ffn(L, W, sel[j], u, h, y);
          for (int64_t c = 0; c < l; ++c) v[c] += g[j] * y[c];
        }
        up_project(L, W, v, out + i * d);
        if (L->n_shared) add_shared(L, W, xt, hs, out + i * d);
      }
    free(xt); free(u); free(z); free(h); free(y); free(v); free(ord); free(asc); free(g);
    free(hs);
  }
  return bad ? -1 : 0;
}

int orc_forward_dense(const orc_layer *L, const orc_weights *W, const void *x,
                      const int64_t *tok, int64_t n, double *out, double *gate_dense) {
  if (check(L, W, x, n) || !out || !gate_dense) return -1;
  const int64_t d = L->d, l = L->l, m = L->m, N = L->n_experts, K = L->top_k;
  int bad = 0;
#pragma omp parallel
  {
    double *xt = malloc(sizeof(double) * (size_t)d);
    double *u = malloc(sizeof(double) * (size_t)(l > d ? l : d));
    double *z = malloc(sizeof(double) * (size_t)N);
    double *h = malloc(sizeof(double) * (size_t)m);
    double *y = malloc(sizeof(double) * (size_t)N * (size_t)l);
    double *v = malloc(sizeof(double) * (size_t)l);
    int32_t *sel = malloc(sizeof(int32_t) * (size_t)K);
    double *g = malloc(sizeof(double) * (size_t)K);
    double *hs = malloc(sizeof(double) * (size_t)(L->m_shared > 0 ? L->m_shared : 1));
    double *ys = malloc(sizeof(double) * (size_t)d);
    const int ok = xt && u && z && h && y && v && sel && g && hs && ys;
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < n; ++i) {
        if (!ok) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        const int64_t t = tok ? tok[i] : i;
        latent_and_logits(L, W, x, t, xt, u, z);
        /* every expert, unconditionally */
        for (int64_t e = 0; e < N; ++e) expert_ffn(L, W, e, u, h, y + e * l);
        /* rank counting: e is chosen iff fewer than K experts beat it */
        int64_t ns = 0;
        for (int64_t e = 0; e < N; ++e) {
          int64_t beat = 0;
          for (int64_t f = 0; f < N; ++f)
            if (z[f] > z[e] || (z[f] == z[e] && f < e)) ++beat;
          if (beat < K && ns < K) sel[ns++] = (int32_t)e;
        }
        gates_for(L, z, sel, ns, g);
        double *G = gate_dense + i * N;
        for (int64_t e = 0; e < N; ++e) G[e] = 0.0;
        for (int64_t j = 0; j < ns; ++j) G[sel[j]] = g[j];
        for (int64_t c = 0; c < l; ++c) v[c] = 0.0;
        for (int64_t e = 0; e < N; ++e)
          for (int64_t c = 0; c < l; ++c) v[c] += G[e] * y[e * l + c];
        up_project(L, W, v, out + i * d);
        /* each shared expert on its own: ys = E_j(x; d), then out += ys */
        const int64_t ms = L->m_shared, H = L->n_shared * ms;
        for (int64_t j = 0; j < L->n_shared; ++j) {
          for (int64_t r = 0; r < ms; ++r) {
            double s = 0.0, sg = 0.0;
            for (int64_t c = 0; c < d; ++c)
              s += ld(W->w_shared1, L->act_dtype, (j * ms + r) * d + c, NULL, 0, NULL) * xt[c];
            if (L->activation == ORC_SWIGLU)
              for (int64_t c = 0; c < d; ++c)
                sg += ld(W->w_shared_gate, L->act_dtype, (j * ms + r) * d + c, NULL, 0, NULL) * xt[c];
            hs[r] = act_fn(L->activation, s, sg);
          }
          for (int64_t r = 0; r < d; ++r) {
            double s = 0.0;
            for (int64_t c = 0; c < ms; ++c)
              s += ld(W->w_shared2, L->act_dtype, r * H + j * ms + c, NULL, 0, NULL) * hs[c];
            ys[r] = s;
          }
          for (int64_t r = 0; r < d; ++r) out[i * d + r] += ys[r];
        }
      }
    free(xt); free(u); free(z); free(h); free(y); free(v); free(sel); free(g); free(hs); free(ys);
  }
  return bad ? -1 : 0;
}

/* Routing alone: for tokens 0 .. n-1, the fp64 router logits (+ bias), the
 * top-K ids ordered by (z desc, id asc) and the margin z_(K) - z_(K+1),
 * exactly as orc_forward takes them, without the experts.  The latent is
 * computed only when the router reads it. */
int orc_route(const orc_layer *L, const orc_weights *W, const void *x, int64_t n, int32_t *idx,
              double *margin, double *logits) {
  if (check(L, W, x, n) || !idx || !margin) return -1;
  const int64_t d = L->d, l = L->l, N = L->n_experts, K = L->top_k;
  int bad = 0;
#pragma omp parallel
  {
    double *xt = malloc(sizeof(double) * (size_t)d);
    double *u = malloc(sizeof(double) * (size_t)(l > d ? l : d));
    double *z = malloc(sizeof(double) * (size_t)N);
    int32_t *ord = malloc(sizeof(int32_t) * (size_t)N);
    const int ok = xt && u && z && ord;
#pragma omp for schedule(dynamic, 4)
      for (int64_t t = 0; t < n; ++t) {
        if (!ok) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        if (L->router_on_latent) {
          input_and_latent(L, W, x, t, xt, u);
        } else {
          for (int64_t c = 0; c < d; ++c) xt[c] = ld(x, L->act_dtype, t * d + c, NULL, 0, NULL);
        }
        router_logits(L, W, xt, u, z);
        if (logits) memcpy(logits + t * N, z, sizeof(double) * (size_t)N);
        sort_by_score(ord, N, z);
        margin[t] = K < N ? z[ord[K - 1]] - z[ord[K]] : INFINITY;
        for (int64_t j = 0; j < K; ++j) idx[t * K + j] = ord[j];
      }
    free(xt); free(u); free(z); free(ord);
  }
  return bad ? -1 : 0;
}

void orc_expert_counts(const int32_t *idx, int64_t n, int64_t K, int64_t N, int64_t *counts) {
  for (int64_t e = 0; e < N; ++e) counts[e] = 0;
  for (int64_t i = 0; i < n * K; ++i)
    if (idx[i] >= 0 && idx[i] < N) ++counts[idx[i]];
}

/* OpenMP threads of the token loops (results do not depend on it). */
void orc_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int orc_max_threads(void) { return omp_get_max_threads(); }
