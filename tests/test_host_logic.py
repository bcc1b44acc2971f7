"""Host-side helpers without a GPU (CPU only): the SwiGLU weight layout,
the attribution of profiled kernels to expert stages, and the workloads'
derived quantities the benchmark uses."""
import numpy as np
import pytest

import mixture_experts_layer_32_amd as pkg
from mixture_experts_layer_32_amd import profiling
from synth import LayerSpec, make_tokens, make_weights, workload


@pytest.mark.parametrize("edt", ["bf16", "fp8_e4m3_rowscale", "mxfp4_e2m1"])
def test_pack_gated_interleaves_rows_numpy_and_torch_alike(edt):
    import torch
    spec = LayerSpec(d=64, l=64, m=32, n_experts=3, top_k=2, expert_dtype=edt,
                     activation="swiglu", n_shared=2, m_shared=32)
    w = make_weights(spec, 4)
    p = pkg.pack_gated(w)
    assert "w_gate" not in p and "w_shared_gate" not in p
    assert np.array_equal(p["w1"][:, 0::2], w["w1"]) and np.array_equal(p["w1"][:, 1::2], w["w_gate"])
    assert np.array_equal(p["w_shared1"][0::2], w["w_shared1"])
    assert np.array_equal(p["w_shared1"][1::2], w["w_shared_gate"])
    for k, g in (("w1_scale", "w_gate_scale"), ("w1_mx", "w_gate_mx")):
        if k in w:
            assert np.array_equal(p[k][:, 0::2], w[k]) and np.array_equal(p[k][:, 1::2], w[g])
    pt = pkg.pack_gated({k: torch.from_numpy(v) for k, v in w.items()})
    for k in p:
        assert np.array_equal(pt[k].numpy(), p[k]), k
    # layers without a gate pass through unchanged
    w0 = make_weights(spec.replace(activation="sqrelu"), 4)
    assert pkg.pack_gated(w0).keys() == w0.keys()


NAMES = {
    "void lmoe::(anonymous namespace)::ffn_stream_kernel<false>(lmoe::FfnArgs)": ("ffn_stream", "ffn"),
    "void lmoe::(anonymous namespace)::gemm_stream_kernel<lmoe::MmaBf16, unsigned short, "
    "unsigned short, unsigned short, 4, 2, 1, false>(lmoe::GemmArgs)": ("gemm_stream", "fc1"),
    "void lmoe::(anonymous namespace)::gemm_stream_kernel<lmoe::MmaBf16, unsigned short, "
    "lmoe::fp4x2_t, unsigned short, 4, 2, 2, false>(lmoe::GemmArgs)": ("gemm_stream", "fc1"),
    "void lmoe::(anonymous namespace)::gemm_stream_kernel<lmoe::MmaBf16, unsigned short, "
    "unsigned char, unsigned short, 8, 1, 0, true>(lmoe::GemmArgs)": ("gemm_stream", "fc2"),
    "void lmoe::(anonymous namespace)::gemm_tiled_kernel<lmoe::MmaBf16x32, unsigned short, "
    "unsigned short, lmoe::TileCfg<128, 256, 2, 2, 4, 3, 2>, 2>"
    "(lmoe::GemmArgs, int, float*)": ("gemm_tiled", "fc1"),
    "void lmoe::(anonymous namespace)::gemm_fp8w_kernel<0, true, true>(lmoe::GemmArgs)":
        ("gemm_fp8w", "fc2"),
    "void lmoe::(anonymous namespace)::gemm_fp8w_kernel<1, true, false>(lmoe::GemmArgs)":
        ("gemm_fp8w", "fc1"),
    "void lmoe::(anonymous namespace)::gemm_tiled_kernel<lmoe::MmaBf16x32, unsigned short, "
    "unsigned short, lmoe::TileCfg<256, 256, 2, 4, 4, 4, 1>, 1>"
    "(lmoe::GemmArgs, int, float*)": ("gemm_tiled", "fc1"),
    "void lmoe::(anonymous namespace)::gemm_grouped_kernel<1, true, false>(lmoe::GemmArgs)":
        ("gemm_grouped", "fc1"),
    "void lmoe::(anonymous namespace)::gemm_grouped_kernel<2, true, false>(lmoe::GemmArgs)":
        ("gemm_grouped", "fc1"),
    "void lmoe::(anonymous namespace)::gemm_grouped_kernel<0, false, false>(lmoe::GemmArgs)":
        ("gemm_grouped", "fc2"),
    # the same kernel as a dense GEMM (W_down, W_up) is not an expert kernel
    "void lmoe::(anonymous namespace)::gemm_grouped_kernel<0, false, true>(lmoe::GemmArgs)":
        (None, None),
    # the same tile without activation is shared with the dense projections
    "void lmoe::(anonymous namespace)::gemm_tiled_kernel<lmoe::MmaBf16x32, unsigned short, "
    "unsigned short, lmoe::TileCfg<256, 256, 2, 4, 4, 4, 1>, 0>"
    "(lmoe::GemmArgs, int, float*)": (None, None),
    # dense GEMMs (projections, router, shared experts) and routing are not expert kernels
    "void lmoe::(anonymous namespace)::gemm_tiled_kernel<lmoe::MmaBf16x32, unsigned short, "
    "float, lmoe::TileCfg<128, 128, 2, 2, 8, 2, 2>, 1>"
    "(lmoe::GemmArgs, int, float*)": (None, None),
    "void lmoe::(anonymous namespace)::combine_kernel<unsigned short, 32>(...)": (None, None),
}


def test_profiled_kernels_map_to_expert_stages():
    for name, (kind, stage) in NAMES.items():
        assert profiling.expert_kernel_kind(name) == kind, name
        assert profiling.expert_stage(name) == stage, name


def test_expert_bytes_per_weight():
    assert workload("latent_decode").spec.expert_bytes == 2
    assert workload("latent_fp8_sparse").spec.expert_bytes == 1
    assert workload("latent_mxfp4_decode").spec.expert_bytes == 0.5 + 1 / 32


def test_table2_variants_follow_the_alpha_rules():
    base = workload("t2_std").spec
    for a in (2, 4, 8):
        s = workload("t2_eff_a%d" % a).spec
        assert (s.l, s.n_experts, s.top_k, s.m) == (base.d // a, base.n_experts * a, base.top_k,
                                                    base.m)
        assert s.l * s.n_experts == base.d * base.n_experts      # same total expert bytes
    acc = workload("t2_acc_a4").spec
    assert acc.top_k * acc.l == base.top_k * base.d                # K' l = K d (Table 1)


def test_latent_router_flag_bound_covers_a_bf16_latent():
    """The parity rule for a router on the bf16-stored latent: a simulated
    kernel (fp32 accumulation of u, RNE to bf16, fp32 logits) stays within
    the shift bound of the fp64 oracle's logits on every token, and every
    token the rule leaves unflagged has the oracle's top-K set."""
    import oracle
    from parity_util import flag_tokens, latent_router_shift_bound
    spec = LayerSpec(d=256, l=96, m=32, n_experts=32, top_k=4, gating="softmax_topk",
                     router_on_latent=True)
    w, x = make_weights(spec, 1), make_tokens(spec, 300, 1)
    f32 = lambda a: oracle.upcast(a, "bf16").astype(np.float32)
    u = f32(x) @ f32(w["w_down"]).T                                # fp32 accumulation
    b = u.view(np.uint32)
    ub = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).view(np.float32)   # RNE to bf16
    z = (ub @ f32(w["w_router"]).T).astype(np.float64)
    tok = np.arange(300)
    ref = oracle.forward(spec, w, x, want_logits=True, want_latent=True)
    bound = latent_router_shift_bound(spec, w, x, tok, ref["latent"])
    assert (np.abs(z - ref["logits"]).max(axis=1) <= bound).all()
    flagged = flag_tokens(spec, w, x, tok, ref)
    sim = np.argsort(-z, axis=1, kind="stable")[:, :spec.top_k]
    same = (np.sort(sim, 1) == np.sort(ref["idx"], 1)).all(1)
    assert same[~flagged].all()
    assert (~flagged).sum() > 0.3 * len(tok)       # the rule still compares most tokens


def test_latent_router_gate_bound_covers_a_bf16_latent():
    """Gates computed from the simulated bf16-latent logits stay within the
    e^(+-2 delta) factor of the oracle's on the unflagged tokens."""
    import oracle
    from parity_util import flag_tokens, latent_router_shift_bound
    spec = LayerSpec(d=256, l=96, m=32, n_experts=32, top_k=4, gating="softmax_topk",
                     router_on_latent=True)
    w, x = make_weights(spec, 1), make_tokens(spec, 200, 1)
    f32 = lambda a: oracle.upcast(a, "bf16").astype(np.float32)
    u = f32(x) @ f32(w["w_down"]).T
    b = u.view(np.uint32)
    ub = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).view(np.float32)
    z = (ub @ f32(w["w_router"]).T).astype(np.float64)
    tok = np.arange(200)
    ref = oracle.forward(spec, w, x, want_logits=True, want_latent=True)
    ok = ~flag_tokens(spec, w, x, tok, ref)
    delta = latent_router_shift_bound(spec, w, x, tok, ref["latent"])
    for t in np.nonzero(ok)[0]:
        ids = ref["idx"][t]
        e = np.exp(z[t, ids] - z[t, ids].max())
        gsim = e / e.sum()
        assert np.all(np.abs(gsim - ref["gate"][t]) <= np.expm1(2 * delta[t]) * ref["gate"][t])
