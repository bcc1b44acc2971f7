"""GPU parity of the SwiGLU experts (W_FC1, W_gate, W_FC2 of LatentMoE §3)
against the fp64 oracle, through the C ABI.

The library reads W_FC1 and W_gate interleaved by rows; the tests pass the
generator's separate matrices through pack_gated.  Small cases run the
oracle on every token for each expert kernel (weight streaming, LDS tiled,
fused decode FFN; bf16, fp8 and fp32 weights), ragged shapes, shared SwiGLU
experts (split-K reduction included) and one token.  Full size: the
LatentMoE variant of the paper's 2048-wide SwiGLU model on sampled tokens.
"""
import numpy as np
import pytest

import synth
from synth import LayerSpec, workload

from parity_util import check_against_oracle, check_routing_structure, run_gpu

pytestmark = pytest.mark.gpu


def _case(spec, T, seed=0):
    return synth.make_weights(spec, seed), synth.make_tokens(spec, T, seed)


def _g(spec, **kw):
    return spec.replace(activation="swiglu", **kw)


CASES = {
    # name: (spec, T, forced expert kernel or None)
    "f32_tiny": (_g(workload("tiny").spec), 64, None),
    "bf16_stream_ragged": (_g(LayerSpec(d=272, l=80, m=208, n_experts=7, top_k=3,
                                        gating="softmax_all")), 133, "stream"),
    "bf16_stream_mb8_zipf": (_g(LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=4,
                                          gating="softmax_all", has_router_bias=True)), 1024,
                             "stream"),
    "bf16_tiled": (_g(LayerSpec(d=256, l=128, m=192, n_experts=8, top_k=2,
                                gating="softmax_topk")), 1000, "tiled"),
    "fp8_tiled": (_g(LayerSpec(d=512, l=128, m=256, n_experts=16, top_k=4, gating="softmax_all",
                               expert_dtype="fp8_e4m3_rowscale")), 200, "tiled"),
    "fp8_stream": (_g(LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=4,
                                gating="sigmoid_topk_norm", expert_dtype="fp8_e4m3_rowscale")),
                   256, "stream"),
    "fused_ragged": (_g(LayerSpec(d=1056, l=1040, m=528, n_experts=24, top_k=4,
                                  gating="sigmoid_topk_norm")), 200, "fused"),
    "fused_multipass": (_g(LayerSpec(d=256, l=128, m=192, n_experts=8, top_k=4,
                                     gating="softmax_topk")), 300, "fused"),
    "fused_m1536": (_g(LayerSpec(d=512, l=256, m=1536, n_experts=300, top_k=2,
                                 gating="softmax_topk")), 600, "fused"),
    "standard_moe_shared": (_g(LayerSpec(d=256, l=256, m=160, n_experts=16, top_k=2,
                                         gating="softmax_all", has_projections=False,
                                         n_shared=1, m_shared=208)), 257, None),
    # shared FC1 with split K: the SwiGLU pairs are formed in the reduction
    "shared_splitk": (_g(LayerSpec(d=2048, l=1040, m=128, n_experts=20, top_k=3,
                                   gating="sigmoid_topk_norm", n_shared=2, m_shared=528)), 100,
                      None),
    "one_token": (_g(LayerSpec(d=256, l=64, m=128, n_experts=16, top_k=4, n_shared=2,
                               m_shared=64)), 1, None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_swiglu_case_matches_oracle(name):
    import mixture_experts_layer_32_amd as pkg
    spec, T, kind = CASES[name]
    layer = pkg.LatentMoELayer(spec, expert_kernel=kind or "auto")
    if kind:  # fp8 experts: the tiled choice is the fp8 register-streaming kernel
        fp8 = spec.expert_dtype == "fp8_e4m3_rowscale"
        assert layer.expert_regime(T) == ("fp8w" if fp8 and kind == "tiled" else kind)
    w, x = _case(spec, T, seed=5)
    g, _ = run_gpu(spec, w, x, layer=layer)
    print(name, "regime", layer.expert_regime(T), flush=True)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g)
    print(name, st, flush=True)


def test_swiglu_expert_kernels_agree():
    import mixture_experts_layer_32_amd as pkg
    spec, T = _g(LayerSpec(d=512, l=256, m=384, n_experts=32, top_k=4,
                           gating="sigmoid_topk_norm")), 256
    w, x = _case(spec, T, seed=3)
    outs = {}
    for kind in ("tiled", "stream", "fused"):
        g, _ = run_gpu(spec, w, x, layer=pkg.LatentMoELayer(spec, expert_kernel=kind))
        outs[kind] = g
    for kind in ("stream", "fused"):
        assert np.array_equal(outs[kind]["topk_idx"], outs["tiled"]["topk_idx"])
        a, b = outs[kind]["out"], outs["tiled"]["out"]
        rel = np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-30)
        assert rel.max() < 2e-2, (kind, rel.max())


def test_unpacked_gate_weights_are_refused():
    import mixture_experts_layer_32_amd as pkg
    spec = _g(LayerSpec(d=256, l=64, m=128, n_experts=16, top_k=4))
    dev = pkg.to_device(synth.make_weights(spec), "cuda:0")
    with pytest.raises(ValueError):
        pkg.LatentMoELayer(spec).weights_struct(dev)


def _sample_tokens(T, n=48, seed=5):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), np.int64)


@pytest.mark.parametrize("kind", ["auto", "fused"])
def test_full_size_swiglu_decode(kind):
    import mixture_experts_layer_32_amd as pkg
    wl = workload("latent_swiglu_decode")
    spec, T = wl.spec, wl.T
    w, x = _case(spec, T, seed=0)
    layer = pkg.LatentMoELayer(spec, expert_kernel=kind)
    g, _ = run_gpu(spec, w, x, layer=layer, overlap=pkg.Overlap())
    print(wl.name, "regime", layer.expert_regime(T), flush=True)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g, tokens=_sample_tokens(T))
    print(wl.name, kind, st, flush=True)
