"""Closed forms of the LatentMoE paper's cost model -- TEST INFRASTRUCTURE ONLY.

LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in Mixture of
Experts:
  §2 (running example): N=128, K=8, d=4096, m=1536, EP=64, F=10 PFLOP/s FP4,
      BW_HBM = 8 TB/s, BW_NVL = 900 GB/s per direction.
  §2.1: compute-bound threshold F/BW_HBM; t_exp = t_total*K/N;
      C_exp = 2 t d m; M_exp = d m + t (d + m) (counted in FP4 "units");
      I = 2 t d m / (d m + t (d + m)) (also the Fig. 2 caption); the
      threshold condition gives t_exp >= 1418.
  §2.2: M_comm = 2.5 (N/EP) t_exp d; C_comp = 2 (N/EP) t_exp d m;
      t_comm / t_comp = 5 F / (4 m BW_NVL), "approximately 9".
  §2.3: binom(aN, aK) >= binom(N, K)^a.
  §3 Table 1: per-GPU communication (N/EP) t_exp {d, l, d} and weight
      loading per expert {d m, l m, d m} for standard / l-MoE_eff / l-MoE_acc
      (the l-MoE_acc row read as per-token totals: K' l m = K d m).
Plus the per-layer FLOP / byte / all-to-all counters of one layer call.
"""
from __future__ import annotations

import math


def compute_bound_threshold(F: float, bw_hbm: float) -> float:
    """F / BW_HBM in FLOP per byte (§2.1)."""
    return F / bw_hbm


def t_exp(t_total: float, K: int, N: int) -> float:
    """Tokens per expert under uniform routing, t_total * K / N (§2.1)."""
    return t_total * K / N


def expert_flops(t: float, d: int, m: int) -> float:
    """C_exp = 2 t d m (§2.1)."""
    return 2.0 * t * d * m


def expert_traffic(t: float, d: int, m: int, bytes_per_elem: float = 1.0) -> float:
    """M_exp = d m + t (d + m) elements, times bytes_per_elem (§2.1)."""
    return bytes_per_elem * (d * m + t * (d + m))


def intensity(t: float, d: int, m: int, bytes_per_elem: float = 1.0) -> float:
    """I = 2 t d m / (d m + t (d + m)) FLOP per byte (§2.1, Fig. 2)."""
    return expert_flops(t, d, m) / expert_traffic(t, d, m, bytes_per_elem)


def min_t_exp(d: int, m: int, threshold: float, bytes_per_elem: float = 1.0) -> float:
    """Exact root of I(t) = threshold: t = thr*b*d*m / (2 d m - thr*b*(d+m))."""
    den = 2.0 * d * m - threshold * bytes_per_elem * (d + m)
    if den <= 0:
        return math.inf
    return threshold * bytes_per_elem * d * m / den


def m_comm(N: int, EP: int, t: float, d: int) -> float:
    """All-to-all bytes per GPU per layer: 2.5 (N/EP) t d (§2.2)."""
    return 2.5 * (N / EP) * t * d


def c_comp(N: int, EP: int, t: float, d: int, m: int) -> float:
    """2 (N/EP) t d m (§2.2)."""
    return 2.0 * (N / EP) * t * d * m


def comm_compute_ratio(F: float, m: int, bw_nvl: float) -> float:
    """t_comm / t_comp = 5 F / (4 m BW_NVL) (§2.2)."""
    return 5.0 * F / (4.0 * m * bw_nvl)


def log10_binom(n: int, k: int) -> float:
    return (math.lgamma(n + 1) - math.lgamma(k + 1) - math.lgamma(n - k + 1)) / math.log(10.0)


def table1(variant: str, N: int, EP: int, t: float, d: int, l: int, m: int, alpha: int = None):
    """(communication cost, weight loading per expert, active experts factor) of Table 1.

    Returns a dict with 'comm' = (N/EP) t_exp w (w = d or l) and
    'weights_per_token' = K_active * w_in * m relative to K of the standard model
    (K_active = K for standard / l-MoE_eff, alpha*K for l-MoE_acc).
    """
    alpha = alpha if alpha is not None else d // l
    if variant == "standard":
        return {"comm_width": d, "weight_per_expert": d * m, "k_factor": 1}
    if variant == "eff":
        return {"comm_width": l, "weight_per_expert": l * m, "k_factor": 1}
    if variant == "acc":
        return {"comm_width": l * alpha, "weight_per_expert": l * m * alpha, "k_factor": alpha}
    raise ValueError(variant)


# ---------------------------------------------------------------------------
# Counters of one layer call (T tokens) for a LayerSpec-like object.

def layer_flops(spec, T: int) -> dict:
    """Algorithmic FLOPs (2 per multiply-add) of each step of one layer call."""
    d, l, m, N, K = spec.d, spec.l, spec.m, spec.n_experts, spec.top_k
    r_in = l if spec.router_on_latent else d
    f = {
        "down": 2.0 * T * d * l if spec.has_projections else 0.0,
        "router": 2.0 * T * r_in * N,
        "fc1": 2.0 * T * K * l * m,
        "fc2": 2.0 * T * K * l * m,
        "up": 2.0 * T * d * l if spec.has_projections else 0.0,
    }
    f["total"] = sum(f.values())
    return f


def layer_bytes(spec, T: int, touched_experts: int) -> dict:
    """Algorithmic HBM bytes of one layer call: weights of the experts that
    received at least one token, projections and router read once, x read
    once, out written once.  Permuted copies, H, Y and logits excluded."""
    d, l, m, N = spec.d, spec.l, spec.m, spec.n_experts
    a = spec.act_bytes
    eb = spec.expert_bytes
    r_in = l if spec.router_on_latent else d
    per_expert = 2.0 * l * m * eb
    if spec.expert_dtype == "fp8_e4m3_rowscale":
        per_expert += 4.0 * (m + l)
    b = {
        "experts": touched_experts * per_expert,
        "proj": (2.0 * l * d * a) if spec.has_projections else 0.0,
        "router": N * r_in * a + (4.0 * N if spec.has_router_bias else 0.0),
        "x": T * d * a,
        "out": T * d * a,
    }
    b["total"] = sum(b.values())
    return b


def a2a_bytes(spec, T: int) -> dict:
    """Bytes an expert-parallel deployment would exchange (not executed here):
    dispatch and combine of T*K latent rows at the activation width, and the
    paper's mixed-precision form 2.5 * T*K*l (FP4 dispatch + BF16 combine)."""
    copies = T * spec.top_k
    return {"dispatch": copies * spec.l * spec.act_bytes,
            "combine": copies * spec.l * spec.act_bytes,
            "paper_fp4_bf16": 2.5 * copies * spec.l}
