"""Pins of the oracle's shared-expert term (CPU only).

The shared experts of LatentMoE Eq. (1)/(2) run ungated on x in the d
space.  The pins tie the term to facts outside the oracle: permutation
weights give a closed form, a shared expert that copies a routed expert of a
standard MoE with gate 1 doubles the output, S = 0 and zero weights drop
the term, and the concatenated evaluation agrees with a per-expert one.
"""
import numpy as np
import pytest

from synth import LayerSpec, make_tokens, make_weights

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _perm_matrix(p):
    """rows r of the result pick element p[r]: (P @ x)[r] = x[p[r]]."""
    P = np.zeros((len(p), len(p)), np.float32)
    P[np.arange(len(p)), p] = 1.0
    return P


def test_permutation_shared_experts_closed_form(orc):
    # Ws1_j = P(pi_j), Ws2_j = P(sigma_j): E_j(x)[r] = max(0, x[pi_j[sigma_j[r]]])^2;
    # pi and sigma are not involutions, so a transposed operand moves the values
    d = 8
    spec = LayerSpec(d=d, l=4, m=8, n_experts=4, top_k=2, gating="softmax_topk",
                     act_dtype="f32", expert_dtype="f32", n_shared=2, m_shared=d)
    pis = [np.array([1, 2, 3, 4, 5, 6, 7, 0]), np.array([3, 0, 6, 1, 7, 2, 5, 4])]
    sigmas = [np.array([2, 0, 1, 5, 3, 4, 7, 6]), np.array([7, 6, 0, 1, 2, 3, 4, 5])]
    w = make_weights(spec, 5)
    w["w_shared1"] = np.concatenate([_perm_matrix(p) for p in pis], axis=0)
    w["w_shared2"] = np.concatenate([_perm_matrix(s) for s in sigmas], axis=1)
    x = make_tokens(spec, 33, 5)
    base = orc.forward(spec.replace(n_shared=0, m_shared=0), w, x)
    got = orc.forward(spec, w, x)
    xs = x.astype(np.float64)
    terms = [np.maximum(0.0, xs[:, p[s]]) ** 2 for p, s in zip(pis, sigmas)]
    # the concatenated sum adds expert 0's one nonzero term, then expert 1's
    assert np.array_equal(got["out"], base["out"] + (terms[0] + terms[1]))
    assert np.array_equal(got["idx"], base["idx"])
    assert np.array_equal(got["gate"], base["gate"])
    dense = orc.forward_dense(spec, w, x)
    np.testing.assert_allclose(dense["out"], got["out"], rtol=1e-14, atol=1e-14)


def test_shared_copy_of_the_only_routed_expert_doubles_output(orc):
    # standard MoE, N = K = 1 (gate exactly 1): a shared expert with the
    # routed expert's weights adds the same value, bit for bit
    d, m = 48, 40
    std = LayerSpec(d=d, l=d, m=m, n_experts=1, top_k=1, gating="softmax_all", act_dtype="f32",
                    expert_dtype="f32", has_projections=False)
    w = make_weights(std, 2)
    x = make_tokens(std, 20, 2)
    base = orc.forward(std, w, x)
    sh = std.replace(n_shared=1, m_shared=m)
    w2 = dict(w, w_shared1=w["w1"][0], w_shared2=w["w2"][0])
    got = orc.forward(sh, w2, x)
    assert np.all(base["gate"] == 1.0)
    assert np.array_equal(got["out"], 2.0 * base["out"])


def test_two_shared_experts_match_two_routed_experts_at_equal_gates(orc):
    # zero router weights give z = 0 for both experts, so each gate is 1/2;
    # shared experts built from the same two FFNs (expert j owning rows
    # j*m of Ws1 and columns j*m of Ws2) add exactly twice the routed term
    d, m = 32, 24
    for gating in ("softmax_all", "softmax_topk", "sigmoid_topk_norm"):
        std = LayerSpec(d=d, l=d, m=m, n_experts=2, top_k=2, gating=gating, act_dtype="f32",
                        expert_dtype="f32", has_projections=False)
        w = make_weights(std, 9)
        w["w_router"] = np.zeros_like(w["w_router"])
        x = make_tokens(std, 25, 9)
        base = orc.forward(std, w, x)
        assert np.all(base["gate"] == 0.5)
        sh = std.replace(n_shared=2, m_shared=m)
        w2 = dict(w, w_shared1=np.concatenate([w["w1"][0], w["w1"][1]], axis=0),
                  w_shared2=np.concatenate([w["w2"][0], w["w2"][1]], axis=1))
        got = orc.forward(sh, w2, x)
        np.testing.assert_allclose(got["out"], 3.0 * base["out"], rtol=1e-12, atol=1e-12)
        # swapping the two shared experts' blocks consistently changes nothing
        w3 = dict(w, w_shared1=np.concatenate([w["w1"][1], w["w1"][0]], axis=0),
                  w_shared2=np.concatenate([w["w2"][1], w["w2"][0]], axis=1))
        np.testing.assert_allclose(orc.forward(sh, w3, x)["out"], got["out"], rtol=1e-12,
                                   atol=1e-12)
        # pairing expert 0's FC1 with expert 1's FC2 does change it
        w4 = dict(w, w_shared1=w2["w_shared1"],
                  w_shared2=np.concatenate([w["w2"][1], w["w2"][0]], axis=1))
        assert not np.allclose(orc.forward(sh, w4, x)["out"], got["out"], rtol=1e-6)


def test_zero_shared_weights_and_zero_S_drop_the_term(orc):
    spec = LayerSpec(d=64, l=16, m=32, n_experts=6, top_k=3, gating="sigmoid_topk_norm",
                     act_dtype="bf16", expert_dtype="bf16", n_shared=2, m_shared=48)
    w = make_weights(spec, 4)
    x = make_tokens(spec, 19, 4)
    base = orc.forward(spec.replace(n_shared=0, m_shared=0), w, x)
    wz = dict(w, w_shared2=np.zeros_like(w["w_shared2"]))
    assert np.array_equal(orc.forward(spec, wz, x)["out"], base["out"])
    # S = 0 ignores whatever shared weights are passed
    assert np.array_equal(orc.forward(spec.replace(n_shared=0), w, x)["out"], base["out"])


SHARED_SPECS = [
    LayerSpec(d=64, l=16, m=32, n_experts=6, top_k=3, gating="sigmoid_topk_norm",
              act_dtype="bf16", expert_dtype="bf16", n_shared=2, m_shared=48),
    LayerSpec(d=48, l=48, m=16, n_experts=5, top_k=2, gating="softmax_all", act_dtype="f32",
              expert_dtype="f32", has_projections=False, n_shared=3, m_shared=16),
    LayerSpec(d=64, l=32, m=16, n_experts=9, top_k=2, gating="softmax_topk", act_dtype="bf16",
              expert_dtype="fp8_e4m3_rowscale", n_shared=1, m_shared=80),
]


@pytest.mark.parametrize("spec", SHARED_SPECS, ids=lambda s: "S%d_ms%d_%s" % (
    s.n_shared, s.m_shared, s.expert_dtype))
def test_concatenated_shared_term_equals_per_expert_sum(orc, spec):
    # the sparse path evaluates the S experts as one concatenated FFN, the
    # dense brute force one expert at a time
    w = make_weights(spec, 7)
    x = make_tokens(spec, 23, 7)
    a = orc.forward(spec, w, x)
    b = orc.forward_dense(spec, w, x)
    scale = np.abs(b["out"]).max()
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-13 * scale)
    base = orc.forward(spec.replace(n_shared=0, m_shared=0), w, x)
    assert np.abs(a["out"] - base["out"]).max() > 1e-3 * scale   # the term is not negligible


def test_shared_needs_weights_and_width(orc):
    spec = LayerSpec(d=64, l=16, m=32, n_experts=6, top_k=3, n_shared=2, m_shared=48)
    w = make_weights(spec, 1)
    x = make_tokens(spec, 3, 1)
    with pytest.raises(ValueError):
        orc.forward(spec.replace(m_shared=0), w, x)
    with pytest.raises(ValueError):
        orc.forward(spec, {k: v for k, v in w.items() if k != "w_shared2"}, x)
