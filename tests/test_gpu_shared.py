"""GPU parity of the shared experts (the second sum of LatentMoE Eq. (1)/(2))
against the fp64 oracle, through the C ABI.

Small cases run the oracle on every token: fp32 and bf16, LatentMoE (the
shared sum added in W_up's epilogue, direct and split-K) and the standard
MoE (added in the combine kernel), shared GEMMs with split K, one token.
The side-stream variant must give bit-identical results to the serial one
(same kernels, same inputs).  Full size: the decode workload with two
shared experts on sampled tokens, in the benchmark's launch configuration.
"""
import numpy as np
import pytest

import synth
from synth import LayerSpec, workload

from parity_util import check_against_oracle, check_routing_structure, run_gpu

pytestmark = pytest.mark.gpu


def _case(spec, T, seed=0):
    return synth.make_weights(spec, seed), synth.make_tokens(spec, T, seed)


SHARED = {
    "tiny_shared_f32": (workload("tiny_shared").spec, 64),
    "bf16_latent_ragged": (LayerSpec(d=272, l=80, m=208, n_experts=7, top_k=3,
                                     gating="softmax_all", n_shared=2, m_shared=96), 133),
    "bf16_standard_moe": (LayerSpec(d=256, l=256, m=160, n_experts=16, top_k=2,
                                    gating="softmax_all", has_projections=False, n_shared=1,
                                    m_shared=208), 257),
    # shared FC1 in 4 K splits (sqrelu in the reduction), FC2 in 2; W_up in
    # 2 K splits (the shared sum added in the reduction)
    "bf16_splitk_everywhere": (LayerSpec(d=2048, l=1040, m=128, n_experts=20, top_k=3,
                                         gating="sigmoid_topk_norm", n_shared=2, m_shared=528),
                               100),
    "fp8_experts_shared": (LayerSpec(d=512, l=128, m=256, n_experts=16, top_k=4,
                                     gating="softmax_all", expert_dtype="fp8_e4m3_rowscale",
                                     n_shared=2, m_shared=128), 200),
    "fused_experts_shared": (LayerSpec(d=512, l=256, m=384, n_experts=300, top_k=2,
                                       gating="softmax_topk", n_shared=3, m_shared=64), 600),
    "one_token": (LayerSpec(d=256, l=64, m=128, n_experts=16, top_k=4, n_shared=2,
                            m_shared=128), 1),
}


@pytest.mark.parametrize("name", list(SHARED))
def test_shared_case_matches_oracle(name):
    spec, T = SHARED[name]
    w, x = _case(spec, T, seed=4)
    g, layer = run_gpu(spec, w, x)
    print(name, "regime", layer.expert_regime(T), flush=True)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g)
    print(name, st, flush=True)


@pytest.mark.parametrize("name", ["bf16_latent_ragged", "bf16_standard_moe",
                                  "bf16_splitk_everywhere", "fused_experts_shared"])
def test_side_stream_is_bit_identical(name):
    import mixture_experts_layer_32_amd as pkg
    spec, T = SHARED[name]
    w, x = _case(spec, T, seed=6)
    layer = pkg.LatentMoELayer(spec)
    a, _ = run_gpu(spec, w, x, layer=layer)
    ov = pkg.Overlap()
    b, _ = run_gpu(spec, w, x, layer=layer, overlap=ov)
    c, _ = run_gpu(spec, w, x, layer=layer, overlap=ov)   # reuse of the events
    for k in a:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k
    ov.close()


def test_shared_term_is_added_once():
    """out(S) - out(S = 0) on the GPU matches the oracle's shared term."""
    spec, T = SHARED["bf16_latent_ragged"]
    w, x = _case(spec, T, seed=7)
    g1, _ = run_gpu(spec, w, x)
    g0, _ = run_gpu(spec.replace(n_shared=0, m_shared=0), w, x)
    import oracle
    r1 = oracle.forward(spec, w, x)["out"]
    r0 = oracle.forward(spec.replace(n_shared=0, m_shared=0), w, x)["out"]
    dg, dr = g1["out"] - g0["out"], r1 - r0
    # both GPU outputs are rounded to bf16: compare against the size of the output
    err = np.linalg.norm(dg - dr, axis=1) / np.maximum(np.linalg.norm(r1, axis=1), 1e-30)
    assert err.max() < 2e-2, err.max()
    assert np.linalg.norm(dr) > 0.1 * np.linalg.norm(r1)


def _sample_tokens(T, n=48, seed=5):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), np.int64)


@pytest.mark.parametrize("overlap", [False, True], ids=["serial", "side_stream"])
def test_full_size_decode_with_shared_experts(overlap):
    import mixture_experts_layer_32_amd as pkg
    wl = workload("latent_decode_shared")
    spec, T = wl.spec, wl.T
    w, x = _case(spec, T, seed=0)
    ov = pkg.Overlap() if overlap else None
    g, layer = run_gpu(spec, w, x, overlap=ov)
    print(wl.name, "regime", layer.expert_regime(T), flush=True)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g, tokens=_sample_tokens(T))
    print(wl.name, "overlap" if overlap else "serial", st, flush=True)


def test_large_tiles_with_shared_experts_sampled():
    """256 x 256 W_up tiles (prefill-sized T) with the shared sum in their
    epilogue, ragged rows and columns."""
    spec, T = LayerSpec(d=2064, l=1040, m=528, n_experts=64, top_k=4, gating="softmax_topk",
                        n_shared=2, m_shared=272), 8200
    w, x = _case(spec, T, seed=8)
    g, _ = run_gpu(spec, w, x)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g, tokens=_sample_tokens(T))
    print("large_tiles_shared", st, flush=True)


def test_stage_timer_and_side_stream_checks():
    """Stage events are recorded as begin/end pairs, the shared stage on the
    side stream; a side stream equal to the launch stream is refused."""
    import torch
    import mixture_experts_layer_32_amd as pkg
    spec, T = SHARED["bf16_latent_ragged"]
    w, x = _case(spec, T, seed=2)
    dev = pkg.to_device(dict(w, x=x), "cuda:0")
    layer = pkg.LatentMoELayer(spec)
    timer = pkg.StageTimer()
    ov = pkg.Overlap()
    for use in (None, ov):
        for _ in range(3):
            layer.forward(dev["x"], dev, timer=timer, overlap=use)
        ms, n = timer.read()
        assert n == 3
        assert set(ms) == set(pkg.STAGE_NAMES)
        assert all(v >= 0 for v in ms.values()), ms
        assert ms["shared"] > 0 and ms["fc1"] > 0 and ms["up"] > 0, ms
    # the null stream is no side stream
    with pytest.raises(pkg.LatentMoEError) as e:
        pkg.Overlap(stream=torch.cuda.default_stream())
    assert e.value.status == -1
    s = torch.cuda.Stream()
    side_on_main = pkg.Overlap(stream=s)
    with pytest.raises(pkg.LatentMoEError) as e:
        layer.forward(dev["x"], dev, overlap=side_on_main, stream=s)
    assert e.value.status == -1
    torch.cuda.synchronize()
    timer.close(); ov.close(); side_on_main.close()
