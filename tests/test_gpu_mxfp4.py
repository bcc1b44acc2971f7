"""GPU parity of MXFP4 expert weights (OCP MX: E2M1 elements, E8M0 scale per
32) against the fp64 oracle, through the C ABI.

Both expert kernels widen each 16-byte chunk (32 elements, one scale
block) to bf16 with the gfx950 scaled conversion (the fused decode FFN
spreads a chunk over two of its stages); the oracle decodes the same codes
exactly.  Small cases: ragged shapes, 64- and 128-row passes,
multi-pass experts under a skewed router, K not a multiple of the 128-element
stage, SwiGLU with shared experts, the standard MoE, one token.  Full size:
the iso-cost LatentMoE decode layer with MXFP4 experts on sampled tokens,
in the fused kernel (AUTO) and the streaming kernel.
"""
import numpy as np
import pytest

import synth
from synth import LayerSpec, workload

from parity_util import check_against_oracle, check_routing_structure, run_gpu

pytestmark = pytest.mark.gpu


def _case(spec, T, seed=0):
    return synth.make_weights(spec, seed), synth.make_tokens(spec, T, seed)


def _mx(spec):
    return spec.replace(expert_dtype="mxfp4_e2m1")


CASES = {
    "ragged_mb8": (_mx(LayerSpec(d=272, l=96, m=224, n_experts=7, top_k=3,
                                 gating="softmax_all")), 133),
    "mb4": (_mx(LayerSpec(d=256, l=128, m=192, n_experts=64, top_k=4,
                          gating="softmax_topk")), 256),
    "zipf_multipass": (_mx(LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=4,
                                     gating="softmax_all", has_router_bias=True)), 1024),
    # K = 160 and 224: the last 128-element stage is partly past K
    "partial_stage": (_mx(LayerSpec(d=512, l=160, m=224, n_experts=16, top_k=4,
                                    gating="sigmoid_topk_norm")), 200),
    "swiglu_shared": (_mx(LayerSpec(d=512, l=128, m=256, n_experts=24, top_k=4,
                                    gating="softmax_all", activation="swiglu", n_shared=2,
                                    m_shared=128)), 300),
    "standard_moe": (_mx(LayerSpec(d=256, l=256, m=160, n_experts=16, top_k=2,
                                   gating="softmax_all", has_projections=False)), 257),
    "one_token": (_mx(LayerSpec(d=256, l=64, m=128, n_experts=16, top_k=4)), 1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mxfp4_case_matches_oracle(name):
    spec, T = CASES[name]
    w, x = _case(spec, T, seed=7)
    g, layer = run_gpu(spec, w, x)
    assert layer.expert_regime(T) == "stream"
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g)
    print(name, st, flush=True)


def test_mxfp4_scale_byte_zero_matches_oracle():
    """E8M0 byte 0 is the subnormal scale 2^-127 (OCP MX): blocks whose scale
    byte is 0, in both expert matrices, decode as in the oracle (their
    elements contribute about 1e-38) and leave the rest of the layer exact."""
    spec, T = CASES["mb4"]
    w, x = _case(spec, T, seed=11)
    for k in ("w1_mx", "w2_mx"):
        sc = w[k].copy()
        sc[:, ::3, 0] = 0          # every third row's first block, every expert
        sc[1::5, :, -1] = 0        # every row's last block of every fifth expert
        w[k] = sc
    g, _ = run_gpu(spec, w, x)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g)
    print("scale_byte_zero", st, flush=True)


def test_mxfp4_equals_bf16_layer_with_decoded_weights():
    """The GPU's MXFP4 layer against its bf16 layer holding the decoded
    weights (exact in bf16): the same routing, outputs within bf16 rounding."""
    import oracle
    spec, T = CASES["mb4"]
    w, x = _case(spec, T, seed=3)
    bf = spec.replace(expert_dtype="bf16")
    wb = {k: v for k, v in w.items() if not k.endswith("_mx")}
    for k in ("w1", "w2"):
        f = oracle.upcast(w[k], "mxfp4_e2m1", w[k + "_mx"]).astype(np.float32)
        wb[k] = (f.view(np.uint32) >> 16).astype(np.uint16)
    a, _ = run_gpu(spec, w, x)
    b, _ = run_gpu(bf, wb, x)
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    rel = np.linalg.norm(a["out"] - b["out"], axis=1) / np.linalg.norm(b["out"], axis=1)
    assert rel.max() < 1e-2, rel.max()


def _sample_tokens(T, n=48, seed=5):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), np.int64)


_FULL = {}


@pytest.mark.parametrize("kernel", ["auto", "stream"])
def test_full_size_mxfp4_decode(kernel):
    """AUTO runs the fused kernel at this size; the streaming kernel forced."""
    import mixture_experts_layer_32_amd as pkg
    wl = workload("latent_mxfp4_decode")
    spec, T = wl.spec, wl.T
    if not _FULL:
        _FULL["wx"] = _case(spec, T, seed=0)
    w, x = _FULL["wx"]
    layer = pkg.LatentMoELayer(spec, expert_kernel=kernel)
    assert layer.expert_regime(T) == ("fused" if kernel == "auto" else "stream")
    g, layer = run_gpu(spec, w, x, layer=layer)
    print(wl.name, "regime", layer.expert_regime(T), flush=True)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g, tokens=_sample_tokens(T))
    print(wl.name, st, flush=True)
    if kernel == "stream":
        _FULL.clear()


# the fused FC1 + FC2 kernel with MXFP4 weights, forced on shapes the
# automatic choice would not give it: ragged l and m (the last 128-element
# double stage partly past K), multi-pass experts with SwiGLU, the widest
# hidden layer, a skewed router with empty experts
FUSED = {
    "fused_ragged": (_mx(LayerSpec(d=1056, l=1056, m=544, n_experts=24, top_k=4,
                                   gating="sigmoid_topk_norm")), 200),
    "fused_multipass_swiglu": (_mx(LayerSpec(d=256, l=128, m=192, n_experts=8, top_k=4,
                                             gating="softmax_topk", activation="swiglu")), 300),
    "fused_m1536": (_mx(LayerSpec(d=512, l=256, m=1536, n_experts=300, top_k=2,
                                  gating="softmax_topk")), 600),
    "fused_zipf_empty": (_mx(LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=4,
                                       gating="softmax_all", has_router_bias=True)), 256),
}


@pytest.mark.parametrize("name", list(FUSED))
def test_mxfp4_fused_matches_oracle(name):
    import mixture_experts_layer_32_amd as pkg
    spec, T = FUSED[name]
    layer = pkg.LatentMoELayer(spec, expert_kernel="fused")
    assert layer.expert_regime(T) == "fused"
    w, x = _case(spec, T, seed=9)
    g, _ = run_gpu(spec, w, x, layer=layer)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g)
    print(name, st, flush=True)


def test_mxfp4_fused_and_stream_agree():
    import mixture_experts_layer_32_amd as pkg
    spec, T = _mx(LayerSpec(d=512, l=256, m=384, n_experts=32, top_k=4,
                            gating="sigmoid_topk_norm")), 256
    w, x = _case(spec, T, seed=3)
    a, _ = run_gpu(spec, w, x, layer=pkg.LatentMoELayer(spec, expert_kernel="fused"))
    b, _ = run_gpu(spec, w, x, layer=pkg.LatentMoELayer(spec, expert_kernel="stream"))
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    rel = np.linalg.norm(a["out"] - b["out"], axis=1) / np.linalg.norm(b["out"], axis=1)
    assert rel.max() < 2e-2, rel.max()
