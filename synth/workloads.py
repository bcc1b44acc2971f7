"""Layer shapes and input recipes of the synthetic workloads.

Shapes follow the LatentMoE paper's running example and deployed models
(LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in Mixture of
Experts, §2 running example: N=128, K=8, d=4096, m=1536; §3 Eq. (2): the
iso-cost variant scales N and K by alpha = d/l) and the secondary article
"Latent MoE 正在成为新的方向" (a 512-expert top-22 model with l = d/4 and an
896-expert top-16 model).  Only shapes and distributions live here.
"""
from __future__ import annotations

import dataclasses


GATINGS = ("softmax_all", "softmax_topk", "sigmoid_topk_norm")
ACTIVATIONS = ("sqrelu", "swiglu")
ACT_DTYPES = ("f32", "bf16")
EXPERT_DTYPES = ("f32", "bf16", "fp8_e4m3_rowscale", "mxfp4_e2m1")


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    d: int
    l: int
    m: int
    n_experts: int
    top_k: int
    gating: str = "softmax_all"
    act_dtype: str = "bf16"
    expert_dtype: str = "bf16"
    has_projections: bool = True
    router_on_latent: bool = False
    has_router_bias: bool = False
    identity_projections: bool = False   # W_down = W_up = I (needs l == d)
    zipf_s: float = 1.1                  # exponent of the log-Zipf router bias
    n_shared: int = 0                    # shared experts S (Eq. (1)/(2)), in the d space
    m_shared: int = 0                    # their hidden width
    activation: str = "sqrelu"           # expert FFN: squared ReLU, or SwiGLU (W_FC1, W_gate, W_FC2)

    def __post_init__(self):
        assert self.gating in GATINGS, self.gating
        assert self.act_dtype in ACT_DTYPES, self.act_dtype
        assert self.expert_dtype in EXPERT_DTYPES, self.expert_dtype
        assert self.activation in ACTIVATIONS, self.activation

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)

    @property
    def act_bytes(self) -> int:
        return 4 if self.act_dtype == "f32" else 2

    @property
    def expert_bytes(self) -> float:
        """Storage bytes per expert weight (MXFP4: half a byte plus a
        one-byte scale per 32 elements)."""
        return {"f32": 4, "bf16": 2, "fp8_e4m3_rowscale": 1,
                "mxfp4_e2m1": 0.5 + 1.0 / 32}[self.expert_dtype]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    spec: LayerSpec
    T: int
    regime: str          # 'tiny', 'decode' (HBM-bound) or 'prefill' (MFMA-bound)
    description: str


WORKLOADS = {
    "tiny": Workload(
        "tiny", LayerSpec(d=256, l=64, m=128, n_experts=16, top_k=4, gating="softmax_topk",
                          act_dtype="f32", expert_dtype="f32"),
        64, "tiny", "tiny LatentMoE, fp32, router on x, softmax over the top-k"),
    "tiny_identity": Workload(
        "tiny_identity", LayerSpec(d=256, l=256, m=128, n_experts=16, top_k=4,
                                   gating="softmax_topk", act_dtype="f32", expert_dtype="f32",
                                   identity_projections=True),
        64, "tiny", "tiny layer with l = d and identity W_down/W_up"),
    "tiny_shared": Workload(
        "tiny_shared", LayerSpec(d=256, l=64, m=128, n_experts=16, top_k=4, gating="softmax_topk",
                                 act_dtype="f32", expert_dtype="f32", n_shared=2, m_shared=64),
        64, "tiny", "tiny LatentMoE with two shared experts in the d space, fp32"),
    "tiny_std": Workload(
        "tiny_std", LayerSpec(d=256, l=256, m=128, n_experts=16, top_k=4, gating="softmax_topk",
                              act_dtype="f32", expert_dtype="f32", has_projections=False),
        64, "tiny", "tiny standard MoE (l = d, no projections)"),
    "std_decode": Workload(
        "std_decode", LayerSpec(d=4096, l=4096, m=1536, n_experts=128, top_k=8,
                                gating="softmax_all", has_projections=False),
        512, "decode", "standard MoE, Qwen3-235B-like shape, bf16, T=512"),
    "latent_decode": Workload(
        "latent_decode", LayerSpec(d=4096, l=1024, m=1536, n_experts=512, top_k=32,
                                   gating="sigmoid_topk_norm"),
        512, "decode", "LatentMoE at iso-cost (alpha=4), bf16, T=512"),
    "latent_decode_shared": Workload(
        "latent_decode_shared", LayerSpec(d=4096, l=1024, m=1536, n_experts=512, top_k=32,
                                          gating="sigmoid_topk_norm", n_shared=2, m_shared=1536),
        512, "decode", "LatentMoE at iso-cost (alpha=4) with S=2 shared experts of width m, "
        "bf16, T=512"),
    "latent_mxfp4_decode": Workload(
        "latent_mxfp4_decode", LayerSpec(d=4096, l=1024, m=1536, n_experts=512, top_k=32,
                                         gating="sigmoid_topk_norm", expert_dtype="mxfp4_e2m1"),
        512, "decode", "LatentMoE at iso-cost (alpha=4), MXFP4 (E2M1 + E8M0 per 32) experts, "
        "bf16 activations, T=512"),
    "latent_swiglu_decode": Workload(
        "latent_swiglu_decode", LayerSpec(d=2048, l=512, m=1408, n_experts=256, top_k=24,
                                          gating="softmax_all", activation="swiglu", n_shared=2,
                                          m_shared=1408),
        512, "decode", "LatentMoE variant of the paper's 2048-wide SwiGLU model (alpha=4: "
        "N 64 -> 256, K 6 -> 24), two shared SwiGLU experts, bf16, T=512"),
    "latent_prefill_zipf": Workload(
        "latent_prefill_zipf", LayerSpec(d=4096, l=1024, m=2048, n_experts=512, top_k=22,
                                         gating="softmax_all", has_router_bias=True),
        16384, "prefill", "512-expert top-22 LatentMoE, bf16, T=16384, log-Zipf(1.1) router bias"),
    "latent_fp8_sparse": Workload(
        "latent_fp8_sparse", LayerSpec(d=7168, l=1792, m=2048, n_experts=896, top_k=16,
                                       gating="softmax_all", expert_dtype="fp8_e4m3_rowscale"),
        4096, "decode", "896-expert top-16 LatentMoE, fp8 e4m3 per-row-scaled experts, bf16 act, T=4096"),
}


# Table 2's 95BT-8BA MoE layer (d 4096, N 128, K 6, S 2 shared experts, m 2688,
# Squared-ReLU) and its LatentMoE variants (§3): l-MoE_eff at alpha = d / l
# keeps K and scales N by alpha (Eq. (1)); l-MoE_acc also scales K (Eq. (2)).
def _table2_95b(alpha: int, acc: bool = False) -> LayerSpec:
    d, N, K, m = 4096, 128, 6, 2688
    if alpha == 1:
        return LayerSpec(d=d, l=d, m=m, n_experts=N, top_k=K, gating="softmax_all",
                         has_projections=False, n_shared=2, m_shared=m)
    return LayerSpec(d=d, l=d // alpha, m=m, n_experts=N * alpha, top_k=K * alpha if acc else K,
                     gating="softmax_all", n_shared=2, m_shared=m)


for _a in (1, 2, 4, 8):
    _n = "t2_std" if _a == 1 else "t2_eff_a%d" % _a
    WORKLOADS[_n] = Workload(
        _n, _table2_95b(_a), 512, "decode",
        "Table 2 95BT-8BA MoE layer" + ("" if _a == 1 else
                                        " as l-MoE_eff, alpha=%d (l %d, N' %d, K 6)"
                                        % (_a, 4096 // _a, 128 * _a)) + ", S=2, bf16, T=512")
WORKLOADS["t2_acc_a4"] = Workload(
    "t2_acc_a4", _table2_95b(4, acc=True), 512, "decode",
    "Table 2 95BT-8BA MoE layer as l-MoE_acc, alpha=4 (l 1024, N' 512, K' 24), S=2, bf16, T=512")


def workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError("unknown workload %r; known: %s" % (name, ", ".join(WORKLOADS)))
