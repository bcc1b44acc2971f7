"""Pins of the oracle's SwiGLU experts (CPU only).

LatentMoE §3 parameterises an expert by W_FC1, W_gate and W_FC2 and Table 2
lists SwiGLU for the 2048-wide model; the reading built is
E(u) = W_FC2 . ((W_FC1 . u) * SiLU(W_gate . u)), SiLU(b) = b * sigmoid(b).
The pins tie it to facts outside the oracle: the sigmoid's closed values at
+-ln 3, +-ln 7 and 0 through selection weights, the limit W_gate = k W_FC1
(k -> inf), where a * SiLU(k a) / k tends to the already pinned squared ReLU,
a zero gate, the dense brute force and a shared copy of a routed expert.
"""
import math

import numpy as np
import pytest

from synth import LayerSpec, make_tokens, make_weights

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

# sigmoid(b) in closed form: 1 / (1 + e^-b) at b = ln q is q / (1 + q)
CLOSED = {0: (math.log(3.0), 0.75), 1: (-math.log(3.0), 0.25), 2: (math.log(7.0), 0.875),
          3: (-math.log(7.0), 0.125), 4: (0.0, 0.5)}


def _sel(idx, n):
    """rows r of the result pick element idx[r]."""
    P = np.zeros((len(idx), n), np.float32)
    P[np.arange(len(idx)), idx] = 1.0
    return P


def test_sigmoid_closed_values_through_selection_weights(orc):
    # identity projections, one expert (gate 1): out = W2 (W1 x * SiLU(Wg x));
    # W1 and W2 are permutations (not involutions), Wg picks only the five
    # entries whose sigmoid has a closed value
    d = 8
    spec = LayerSpec(d=d, l=d, m=d, n_experts=1, top_k=1, gating="softmax_all", act_dtype="f32",
                     expert_dtype="f32", identity_projections=True, activation="swiglu")
    w = make_weights(spec, 3)
    p1 = np.array([5, 0, 7, 1, 6, 2, 3, 4])
    q = np.array([0, 2, 4, 1, 3, 0, 3, 2])
    p3 = np.array([1, 2, 3, 4, 5, 6, 7, 0])
    w["w1"] = _sel(p1, d)[None]
    w["w_gate"] = _sel(q, d)[None]
    w["w2"] = _sel(p3, d)[None]
    rng = np.random.default_rng(0)
    rows = []
    for _ in range(6):
        row = np.empty(d, np.float32)
        row[:5] = [CLOSED[i][0] for i in range(5)]
        row[5:] = rng.standard_normal(3).astype(np.float32)
        rows.append(row)
    x = np.stack(rows)
    got = orc.forward(spec, w, x)["out"]
    xs = x.astype(np.float64)
    sig = np.array([CLOSED[i][1] for i in q])
    h = xs[:, p1] * xs[:, q] * sig[None, :]
    want = h[:, p3]
    # the stored float32 ln q differ from ln q by < 2^-24 relative
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-12)


@pytest.mark.parametrize("edt", ["f32", "bf16", "fp8_e4m3_rowscale"])
def test_large_gate_scale_tends_to_squared_relu(orc, edt):
    # W_gate = k W_FC1: a * SiLU(k a) / k = a^2 sigmoid(k a), which differs
    # from max(0, a)^2 by at most a^2 sigmoid(-k |a|) <= (2 / (e k))^2
    act = "f32" if edt == "f32" else "bf16"
    base = LayerSpec(d=96, l=48, m=64, n_experts=6, top_k=3, gating="softmax_topk",
                     act_dtype=act, expert_dtype=edt)
    sw = base.replace(activation="swiglu")
    w = make_weights(sw, 11)
    x = make_tokens(sw, 21, 11)
    k = 4096.0
    if edt == "fp8_e4m3_rowscale":
        w["w_gate"], w["w_gate_scale"] = w["w1"].copy(), w["w1_scale"] * np.float32(k)
    elif edt == "bf16":
        g = (w["w1"].astype(np.uint32) << 16).view(np.float32) * np.float32(k)   # exact: power of 2
        w["w_gate"] = (g.view(np.uint32) >> 16).astype(np.uint16)
    else:
        w["w_gate"] = w["w1"] * np.float32(k)
    ref = orc.forward(base, w, x)
    got = orc.forward(sw, w, x)
    assert np.array_equal(got["idx"], ref["idx"])
    scale = np.abs(ref["out"]).max()
    np.testing.assert_allclose(got["out"] / k, ref["out"], rtol=0, atol=1e-6 * scale)


def test_zero_gate_gives_zero_experts(orc):
    spec = LayerSpec(d=64, l=64, m=32, n_experts=5, top_k=2, gating="softmax_all",
                     act_dtype="f32", expert_dtype="f32", has_projections=False,
                     activation="swiglu")
    w = make_weights(spec, 2)
    w["w_gate"] = np.zeros_like(w["w_gate"])
    x = make_tokens(spec, 9, 2)
    assert np.array_equal(orc.forward(spec, w, x)["out"], np.zeros((9, 64)))


SPECS = [
    LayerSpec(d=64, l=32, m=48, n_experts=7, top_k=3, gating="softmax_all", act_dtype="bf16",
              expert_dtype="bf16", activation="swiglu", has_router_bias=True),
    LayerSpec(d=64, l=32, m=16, n_experts=9, top_k=2, gating="sigmoid_topk_norm",
              act_dtype="bf16", expert_dtype="fp8_e4m3_rowscale", activation="swiglu"),
    LayerSpec(d=32, l=32, m=24, n_experts=4, top_k=4, gating="softmax_topk", act_dtype="f32",
              expert_dtype="f32", has_projections=False, activation="swiglu"),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: "N%dK%d_%s" % (s.n_experts, s.top_k,
                                                                     s.expert_dtype))
def test_sparse_equals_dense_bruteforce_bit_exact(orc, spec):
    w = make_weights(spec, 4)
    x = make_tokens(spec, 29, 4)
    a = orc.forward(spec, w, x)
    b = orc.forward_dense(spec, w, x)
    assert np.array_equal(a["out"], b["out"])


def test_shared_swiglu_copy_of_the_only_routed_expert_doubles_output(orc):
    d, m = 48, 40
    std = LayerSpec(d=d, l=d, m=m, n_experts=1, top_k=1, gating="softmax_all", act_dtype="f32",
                    expert_dtype="f32", has_projections=False, activation="swiglu")
    w = make_weights(std, 6)
    x = make_tokens(std, 15, 6)
    base = orc.forward(std, w, x)
    sh = std.replace(n_shared=1, m_shared=m)
    w2 = dict(w, w_shared1=w["w1"][0], w_shared2=w["w2"][0], w_shared_gate=w["w_gate"][0])
    assert np.array_equal(orc.forward(sh, w2, x)["out"], 2.0 * base["out"])
    # a shared gate taken from the wrong matrix changes the result
    w3 = dict(w2, w_shared_gate=w["w1"][0])
    assert not np.allclose(orc.forward(sh, w3, x)["out"], 2.0 * base["out"], rtol=1e-3)


def test_swiglu_needs_its_gate_weights(orc):
    spec = LayerSpec(d=64, l=16, m=32, n_experts=6, top_k=3, activation="swiglu", n_shared=1,
                     m_shared=16)
    w = make_weights(spec, 1)
    x = make_tokens(spec, 3, 1)
    for k in ("w_gate", "w_shared_gate"):
        with pytest.raises(ValueError):
            orc.forward(spec, {kk: v for kk, v in w.items() if kk != k}, x)
