"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Small cases run the oracle on every token and span several tiles with
ragged tails (T, N, d, l, m not multiples of the tile sizes), both expert
kernels (weight-streaming and LDS-tiled), fp32 / bf16 / fp8 weights, the
three gating rules, router bias, router on the latent, the standard MoE and
degenerate shapes.  Full-size cases run the shapes of the benchmark
workloads in the same launch configuration as bench.py and compare sampled
tokens one by one, plus the routing invariants for every token.
"""
import numpy as np
import pytest

import synth
from synth import LayerSpec, workload

from parity_util import (check_against_oracle, check_routing_all_tokens,
                         check_routing_structure, run_gpu)

pytestmark = pytest.mark.gpu


def _case(spec, T, seed=0):
    return synth.make_weights(spec, seed), synth.make_tokens(spec, T, seed)


SMALL = {
    "tiny_f32": (workload("tiny").spec, 64),
    "tiny_f32_sigmoid_latent_router": (workload("tiny").spec.replace(
        gating="sigmoid_topk_norm", router_on_latent=True), 64),
    "bf16_ragged_stream_mb8": (LayerSpec(d=272, l=80, m=208, n_experts=7, top_k=3,
                                         gating="softmax_all"), 133),
    "bf16_sigmoid_stream": (LayerSpec(d=512, l=128, m=320, n_experts=24, top_k=5,
                                      gating="sigmoid_topk_norm"), 300),
    "bf16_stream_mb4": (LayerSpec(d=256, l=128, m=192, n_experts=64, top_k=4,
                                  gating="softmax_topk"), 256),
    "bf16_tiled_experts": (LayerSpec(d=256, l=128, m=192, n_experts=8, top_k=2,
                                     gating="softmax_topk"), 1000),
    "bf16_zipf_bias_tiled": (LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=6,
                                       gating="softmax_all", has_router_bias=True), 2048),
    "bf16_zipf_bias_stream_multipass": (LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=4,
                                                  gating="softmax_all", has_router_bias=True),
                                        1024),
    "bf16_latent_router": (LayerSpec(d=256, l=96, m=128, n_experts=32, top_k=4,
                                     gating="softmax_topk", router_on_latent=True), 200),
    "bf16_standard_moe": (LayerSpec(d=256, l=256, m=160, n_experts=16, top_k=2,
                                    gating="softmax_all", has_projections=False), 257),
    "fp8_tiled": (LayerSpec(d=512, l=128, m=256, n_experts=16, top_k=4,
                            gating="softmax_all", expert_dtype="fp8_e4m3_rowscale"), 200),
    "fp8_tiled_many_rows": (LayerSpec(d=256, l=160, m=288, n_experts=8, top_k=2,
                                      gating="softmax_topk", expert_dtype="fp8_e4m3_rowscale"),
                            1000),
    "fp8_zipf_stream_multipass": (LayerSpec(d=256, l=96, m=160, n_experts=32, top_k=3,
                                            gating="softmax_all", expert_dtype="fp8_e4m3_rowscale",
                                            has_router_bias=True), 400),
    "fp8_stream_mb4": (LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=4,
                                 gating="sigmoid_topk_norm", expert_dtype="fp8_e4m3_rowscale"), 256),
    "fp8_zipf_multipass": (LayerSpec(d=256, l=96, m=160, n_experts=32, top_k=3,
                                     gating="softmax_all", expert_dtype="fp8_e4m3_rowscale",
                                     has_router_bias=True), 700),
    "f32_tiled_experts": (LayerSpec(d=128, l=64, m=96, n_experts=4, top_k=2,
                                    gating="softmax_all", act_dtype="f32", expert_dtype="f32"), 600),
    # dense GEMMs split K in two (17 stages: 9 + 8) and reduce the fp32 partials
    "bf16_splitk_ragged": (LayerSpec(d=1040, l=64, m=128, n_experts=20, top_k=3,
                                     gating="softmax_all"), 100),
    "one_token": (LayerSpec(d=256, l=64, m=128, n_experts=16, top_k=4), 1),
    "k_equals_n": (LayerSpec(d=128, l=64, m=64, n_experts=8, top_k=8, gating="softmax_all"), 40),
    "single_expert": (LayerSpec(d=128, l=64, m=64, n_experts=1, top_k=1), 50),
    "k64_n128": (LayerSpec(d=128, l=64, m=64, n_experts=128, top_k=64, gating="sigmoid_topk_norm"), 30),
    "n2048": (LayerSpec(d=128, l=64, m=64, n_experts=2048, top_k=16), 64),
    # the largest N with the largest K: the top-k search fills all 64 lanes
    "n2048_k64": (LayerSpec(d=128, l=64, m=64, n_experts=2048, top_k=64,
                            gating="sigmoid_topk_norm"), 70),
    # W_down and the router in one launch over x on 128 x 128 tiles with K
    # split in two (the fp32-output plan for 128-255 such tiles), the top-k
    # kernel finishing u from the partials
    "front_tile128_split": (LayerSpec(d=1024, l=512, m=128, n_experts=2048, top_k=8,
                                      gating="softmax_all"), 832),
    # dispatch in three kernels, the column scan over 300 experts (a last
    # workgroup of 44) and 32 token blocks
    "route_scan_n300": (LayerSpec(d=256, l=64, m=128, n_experts=300, top_k=6,
                                  gating="softmax_all", has_router_bias=True), 2000),
    # the column scan over 313 token blocks (its waves take 20 blocks each:
    # two full batches of 8 and a remainder of 4)
    "route_scan_313_blocks": (LayerSpec(d=256, l=256, m=256, n_experts=40, top_k=2,
                                        gating="softmax_topk"), 20000),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_case_matches_oracle(name):
    spec, T = SMALL[name]
    w, x = _case(spec, T, seed=1)
    g, layer = run_gpu(spec, w, x)
    print(name, "regime", layer.expert_regime(T), flush=True)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g)
    print(name, st, flush=True)


# Each expert kernel forced on shapes the automatic choice would not give it.
FORCED = {
    # fused FC1 + FC2: ragged l and m (last tiles partial, stages padded),
    # fewer experts than compute units
    "fused_ragged": (LayerSpec(d=1056, l=1040, m=528, n_experts=24, top_k=4,
                               gating="sigmoid_topk_norm"), 200, "fused"),
    # experts with several 48-row passes
    "fused_multipass": (LayerSpec(d=256, l=128, m=192, n_experts=8, top_k=4,
                                  gating="softmax_topk"), 300, "fused"),
    # skewed loads: empty experts and multi-pass ones in one batch
    "fused_zipf_empty": (LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=4,
                                   gating="softmax_all", has_router_bias=True), 256, "fused"),
    # the largest hidden width that fits on chip, more experts than compute units
    "fused_m1536": (LayerSpec(d=512, l=256, m=1536, n_experts=300, top_k=2,
                              gating="softmax_topk"), 600, "fused"),
    "fused_one_token": (LayerSpec(d=256, l=64, m=128, n_experts=16, top_k=4), 1, "fused"),
    "tiled_few_rows": (LayerSpec(d=256, l=128, m=192, n_experts=64, top_k=4,
                                 gating="softmax_topk"), 256, "tiled"),
    "stream_many_rows": (LayerSpec(d=256, l=128, m=192, n_experts=8, top_k=2,
                                   gating="softmax_topk"), 1000, "stream"),
    # the streaming kernel's 128-row passes (more than 40 rows per expert)
    # and multi-pass experts, on shapes the automatic choice gives to the
    # tiled kernel
    "stream_mb8_ragged": (LayerSpec(d=272, l=80, m=208, n_experts=7, top_k=3,
                                    gating="softmax_all"), 133, "stream"),
    "stream_sigmoid_mb8": (LayerSpec(d=512, l=128, m=320, n_experts=24, top_k=5,
                                     gating="sigmoid_topk_norm"), 300, "stream"),
    "stream_zipf_multipass": (LayerSpec(d=256, l=64, m=128, n_experts=64, top_k=4,
                                        gating="softmax_all", has_router_bias=True), 1024,
                              "stream"),
    # sparse batch (1 copy per expert on average): the streaming kernel works
    # from the dispatch stage's list of experts with copies; the skewed
    # router still gives some experts several passes
    "stream_sparse_zipf": (LayerSpec(d=512, l=128, m=192, n_experts=512, top_k=4,
                                     gating="softmax_all", has_router_bias=True), 128, "stream"),
    "stream_sparse_fp8": (LayerSpec(d=256, l=64, m=128, n_experts=256, top_k=2,
                                    gating="sigmoid_topk_norm", expert_dtype="fp8_e4m3_rowscale"),
                          100, "stream"),
    # sparse, with the dispatch in three kernels (4 token blocks x 2048 experts
    # exceed the single-workgroup route): the scan kernel writes the list
    "stream_sparse_route_scan": (LayerSpec(d=256, l=64, m=128, n_experts=2048, top_k=8,
                                           gating="softmax_all"), 200, "stream"),
}


@pytest.mark.parametrize("name", list(FORCED))
def test_forced_expert_kernel_matches_oracle(name):
    import mixture_experts_layer_32_amd as pkg
    spec, T, kind = FORCED[name]
    layer = pkg.LatentMoELayer(spec, expert_kernel=kind)
    assert layer.expert_regime(T) == kind
    w, x = _case(spec, T, seed=2)
    g, _ = run_gpu(spec, w, x, layer=layer)
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g)
    print(name, kind, st, flush=True)


def test_expert_kernels_agree():
    """The three expert kernels on one input: same routing, outputs within
    the bf16 tolerance of each other (each is checked against the oracle
    above)."""
    import mixture_experts_layer_32_amd as pkg
    spec, T = LayerSpec(d=512, l=256, m=384, n_experts=32, top_k=4,
                        gating="sigmoid_topk_norm"), 256
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


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_identity_projections_equal_standard_moe_bit_exact(act):
    base = workload("tiny_identity").spec.replace(act_dtype=act, expert_dtype=act)
    std = base.replace(has_projections=False, identity_projections=False)
    w, x = _case(base, 64)
    w_std = {k: v for k, v in w.items() if k not in ("w_down", "w_up")}
    a, _ = run_gpu(base, w, x)
    b, _ = run_gpu(std, w_std, x)
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    assert np.array_equal(a["out"], b["out"])
    # W_down = I: the stored latent is x itself, bit for bit
    xv = x.astype(np.float64) if act == "f32" else \
        (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(a["latent"], xv)
    check_against_oracle(std, w_std, x, b)


def test_repeated_calls_are_bit_identical():
    spec, T = SMALL["bf16_zipf_bias_tiled"]
    w, x = _case(spec, T)
    a, layer = run_gpu(spec, w, x)
    b, _ = run_gpu(spec, w, x, layer=layer)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_zero_tokens_is_a_noop():
    import torch
    import mixture_experts_layer_32_amd as pkg
    spec = workload("tiny").spec
    layer = pkg.LatentMoELayer(spec)
    dev = pkg.to_device(synth.make_weights(spec), "cuda:0")
    x = torch.empty((0, spec.d), dtype=torch.float32, device="cuda:0")
    out = layer.forward(x, dev)
    assert out.shape == (0, spec.d)


# ---------------------------------------------------------------- full size

FULL = ["std_decode", "latent_decode", "latent_prefill_zipf", "latent_fp8_sparse"]


def _sample_tokens(T, n=48, seed=5):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), np.int64)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_tokens(name):
    wl = workload(name)
    spec, T = wl.spec, wl.T
    w, x = _case(spec, T, seed=0)
    g, layer = run_gpu(spec, w, x)
    print(name, "regime", layer.expert_regime(T), flush=True)
    check_routing_structure(spec, g, T)
    # every token: ids (unflagged) and per-expert counts bit-exact, logits
    rt = check_routing_all_tokens(spec, w, x, g)
    print(name, "routing", rt, flush=True)
    # outputs on 128 sampled tokens plus the first and last (the last dense
    # row tile)
    st = check_against_oracle(spec, w, x, g, tokens=_sample_tokens(T, n=128))
    print(name, st, flush=True)


def _tie_router(N, d, scen):
    """Router rows and one-hot token columns so that every logit is an exact
    small integer (sums of a few +-1, 2, 3 terms: no rounding in any order).
    Scenario s uses column s of x; the values a_s[e] are W_r[e][s]."""
    wr = np.zeros((N, d), np.float32)
    for s, vals in enumerate(scen):
        wr[:, s] = vals
    return wr


def _tie_scenarios(N, K, rng):
    sc = [np.zeros(N)]                                        # all-zero router
    a = np.zeros(N); a[rng.choice(N, 1)] = 3.0                 # one leader, then
    tied = rng.choice(np.setdiff1d(np.arange(N), np.nonzero(a)[0]), K + 2, replace=False)
    a[tied] = 2.0; sc.append(a)                                # K + 2 tied across the K-th place
    b = np.full(N, -1.0); b[rng.choice(N, K + 5, replace=False)] = 1.0
    sc.append(b)                                               # K + 5 tied at the top
    c = rng.integers(-2, 3, N).astype(np.float64); sc.append(c)  # many ties everywhere
    e = np.zeros(N); e[-(K - 1):] = 1.0; sc.append(e)          # top K-1 at the highest ids,
    return sc                                                  # the rest from the zeros


@pytest.mark.parametrize("N,K,gating", [(32, 4, "softmax_all"), (200, 6, "sigmoid_topk_norm"),
                                        (512, 22, "softmax_topk"), (2048, 16, "softmax_all")])
def test_crafted_ties_go_to_the_lower_expert_id(N, K, gating):
    """Exact logit ties on the GPU (the kernel's single- and multi-holder
    branches, ties within a lane and across lanes): the set taken is the K
    best under (logit desc, id asc), fixed by construction."""
    rng = np.random.default_rng(N + K)
    spec = LayerSpec(d=128, l=64, m=64, n_experts=N, top_k=K, gating=gating)
    scen = _tie_scenarios(N, K, rng)
    w = synth.make_weights(spec, 0)
    wr = _tie_router(N, spec.d, scen)
    w = dict(w, w_router=(wr.view(np.uint32) >> 16).astype(np.uint16))   # exact in bf16
    T = 4 * len(scen)
    x32 = np.zeros((T, spec.d), np.float32)
    for t in range(T):
        x32[t, t % len(scen)] = 1.0
    x = (x32.view(np.uint32) >> 16).astype(np.uint16)
    g, _ = run_gpu(spec, w, x)
    check_routing_structure(spec, g, T)
    for t in range(T):
        z = wr[:, t % len(scen)].astype(np.float64)
        want = sorted(np.lexsort((np.arange(N), -z))[:K].tolist())
        assert sorted(g["topk_idx"][t].tolist()) == want, (t, scen[t % len(scen)][:8])
        assert np.array_equal(g["logits"][t], z.astype(np.float32))
    # the oracle takes the same sets, and the outputs agree (every token is
    # flagged, margin 0, so outputs are compared with the GPU's sets)
    ref = __import__("oracle").route(spec, w, x)
    assert np.array_equal(np.sort(ref["idx"], 1), np.sort(g["topk_idx"], 1))
    check_against_oracle(spec, w, x, g)


# The persistent grouped kernel (experts with 256 rows or more on average):
# skewed loads give every tile height (256, 128, 64 rows), experts with no
# rows and experts of many full tiles in one launch; SwiGLU, the standard
# MoE and a single expert.
GROUPED = {
    "grouped_zipf": (LayerSpec(d=512, l=256, m=512, n_experts=8, top_k=2, gating="softmax_all",
                               has_router_bias=True), 1500),
    "grouped_swiglu": (LayerSpec(d=256, l=256, m=256, n_experts=4, top_k=2, gating="softmax_topk",
                                 activation="swiglu"), 700),
    "grouped_std_moe": (LayerSpec(d=512, l=512, m=256, n_experts=4, top_k=1, gating="softmax_all",
                                  has_projections=False), 1200),
    "grouped_one_expert": (LayerSpec(d=256, l=256, m=512, n_experts=1, top_k=1), 300),
    "grouped_many_experts_zipf": (LayerSpec(d=256, l=256, m=256, n_experts=64, top_k=8,
                                            gating="softmax_all", has_router_bias=True), 2100),
}


@pytest.mark.parametrize("name", list(GROUPED))
def test_grouped_kernel_matches_oracle(name):
    import mixture_experts_layer_32_amd as pkg
    spec, T = GROUPED[name]
    layer = pkg.LatentMoELayer(spec)
    assert layer.expert_regime(T) == "grouped"
    w, x = _case(spec, T, seed=4)
    g, _ = run_gpu(spec, w, x, layer=layer)
    counts = g["expert_counts"]
    print(name, "rows per expert", counts.tolist(), flush=True)
    check_routing_structure(spec, g, T)
    tok = None if T * spec.top_k * spec.m * spec.l <= 2e9 else _sample_tokens(T, n=200, seed=7)
    st = check_against_oracle(spec, w, x, g, tokens=tok)
    print(name, st, flush=True)


@pytest.mark.parametrize("name", ["grouped_zipf", "grouped_swiglu", "grouped_std_moe",
                                  "grouped_many_experts_zipf"])
def test_grouped_packed_weights_bit_identical(name):
    """The banded copy of W1 and W2 (latentmoe_pack_expert_weights) changes
    only where the grouped kernel reads each weight stage: the outputs are
    bit-identical to the row-major run, and match the oracle."""
    import mixture_experts_layer_32_amd as pkg
    spec, T = GROUPED[name]
    layer = pkg.LatentMoELayer(spec)
    assert layer.packed_weights_size() > 0 and layer.expert_regime(T) == "grouped"
    w, x = _case(spec, T, seed=4)
    a, _ = run_gpu(spec, w, x, layer=layer)
    b, _ = run_gpu(spec, w, x, layer=layer, packed=True)
    assert np.array_equal(a["out"], b["out"])
    tok = None if T * spec.top_k * spec.m * spec.l <= 2e9 else _sample_tokens(T, n=200, seed=7)
    st = check_against_oracle(spec, w, x, b, tokens=tok)
    print(name, st, flush=True)


@pytest.mark.parametrize("spec,T", [
    (LayerSpec(d=512, l=256, m=384, n_experts=8, top_k=2, gating="softmax_all",
               expert_dtype="fp8_e4m3_rowscale"), 400),
    (LayerSpec(d=256, l=128, m=192, n_experts=6, top_k=2, gating="softmax_topk",
               activation="swiglu", expert_dtype="fp8_e4m3_rowscale"), 500),
], ids=["fp8", "fp8_swiglu"])
def test_fp8_packed_weights_bit_identical(spec, T):
    """fp8 experts with the banded copy (16-row bands) in the fp8 kernel:
    bit-identical to the row-major run, and matching the oracle."""
    import mixture_experts_layer_32_amd as pkg
    layer = pkg.LatentMoELayer(spec)
    assert layer.packed_weights_size() > 0 and layer.expert_regime(T) == "fp8w"
    w, x = _case(spec, T, seed=6)
    a, _ = run_gpu(spec, w, x, layer=layer)
    b, _ = run_gpu(spec, w, x, layer=layer, packed=True)
    assert np.array_equal(a["out"], b["out"])
    st = check_against_oracle(spec, w, x, b)
    print(spec.activation, st, flush=True)


@pytest.mark.parametrize("name", ["latent_prefill_zipf", "latent_fp8_sparse"])
def test_full_size_packed_weights_bit_identical(name):
    """The prefill and fp8 layers with the banded expert weights, as the
    benchmark runs them: bit-identical to the row-major run (which the
    full-size test above checks against the oracle)."""
    wl = workload(name)
    spec, T = wl.spec, wl.T
    w, x = _case(spec, T, seed=0)
    a, layer = run_gpu(spec, w, x)
    assert layer.expert_regime(T) in ("grouped", "fp8w")
    b, _ = run_gpu(spec, w, x, layer=layer, packed=True)
    assert np.array_equal(a["out"], b["out"])


# Sizes that select (256 x 256 dense, 128 x 256 grouped,
# 128 x 128 dense) with ragged row and column tails, on sampled tokens.
# ragged_dense_grouped: enough rows for W_down and W_up to run in the
# persistent grouped kernel as one group (256 x 256 tiles, at least one per
# compute unit), the last row tile 188 rows high; the experts run grouped too.
MID = {
    "ragged_large_tiles": (LayerSpec(d=2064, l=1040, m=528, n_experts=64, top_k=4,
                                     gating="softmax_topk"), 8200, "tiled"),
    "ragged_dense_grouped": (LayerSpec(d=2048, l=512, m=512, n_experts=32, top_k=4,
                                       gating="softmax_topk"), 32700, "grouped"),
    # expert GEMMs only on the grouped kernel (W_down / W_up too small for it)
    # with several items per compute unit: FC1 about 580, FC2 about 290
    # (expert, row tile, column tile) items over the 256 workgroups, so each
    # workgroup walks more than one tile and tile heights change along a walk
    "grouped_many_items": (LayerSpec(d=512, l=512, m=1024, n_experts=16, top_k=4,
                                     gating="softmax_all", has_router_bias=True), 8191, "grouped"),
}


@pytest.mark.parametrize("name", sorted(MID))
def test_mid_size_large_tiles_sampled_tokens(name):
    spec, T, regime = MID[name]
    w, x = _case(spec, T, seed=3)
    g, layer = run_gpu(spec, w, x)
    assert layer.expert_regime(T) == regime
    check_routing_structure(spec, g, T)
    st = check_against_oracle(spec, w, x, g, tokens=_sample_tokens(T, n=40, seed=9))
    print(name, st, flush=True)



def test_one_handle_on_two_streams_at_once():
    """The handle is immutable: two calls in flight on two streams, each with
    its own workspace and output, give the results of separate calls."""
    import torch
    import mixture_experts_layer_32_amd as pkg
    spec, T = SMALL["bf16_zipf_bias_tiled"]
    layer = pkg.LatentMoELayer(spec)
    w = synth.make_weights(spec, 0)
    dev = pkg.to_device(w, "cuda:0")
    xs = [pkg.to_device({"x": synth.make_tokens(spec, T, seed)}, "cuda:0")["x"] for seed in (1, 2)]
    ref = []
    for x in xs:
        ref.append(layer.forward(x, dev).clone())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(r) for r in ref]
    wss = [torch.empty((layer.workspace_size(T),), dtype=torch.uint8, device="cuda:0")
           for _ in xs]
    cw = layer.weights_struct(dev)
    for _ in range(3):
        for x, o, ws, st in zip(xs, outs, wss, streams):
            layer.forward(x, None, out=o, workspace=ws, cweights=cw, stream=st)
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert torch.equal(o, r)
