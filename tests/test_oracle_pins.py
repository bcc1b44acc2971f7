"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties the oracle to something the pages or the mathematics fix:
the identity reduction (l = d with W_down = W_up = I is the standard MoE),
a brute-force dense evaluation with rank-counting selection, textbook
special cases (N = K = 1 is a plain two-layer Squared-ReLU MLP; K = N with
softmax gating is a dense softmax mixture), invariants of routing and gating,
crafted ties, and the exact storage formats.  A dropped term, a wrong index,
a transposed operand or a wrong gate fails at least one of them.
"""
import math

import numpy as np
import pytest
from scipy.special import expit, softmax

from synth import LayerSpec, make_tokens, make_weights, workload

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _inputs(spec, T, seed=0):
    return make_weights(spec, seed), make_tokens(spec, T, seed)


def _f64(orc, spec, w, key):
    dt = spec.act_dtype if key in ("w_down", "w_up", "w_router") else spec.expert_dtype
    scale = w.get(key + "_scale")
    return orc.upcast(w[key], dt, scale)


# --------------------------------------------------------------------------
# identity reduction: l = d, W_down = W_up = I  ==  standard MoE, bit-exact

@pytest.mark.parametrize("gating", ["softmax_all", "softmax_topk", "sigmoid_topk_norm"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_identity_projection_reduces_to_standard_moe_bit_exact(orc, gating, act):
    base = workload("tiny_identity").spec.replace(gating=gating, act_dtype=act,
                                                  expert_dtype=act)
    std = base.replace(has_projections=False, identity_projections=False)
    w_id, x = _inputs(base, 64)
    w_std = {k: v for k, v in w_id.items() if k not in ("w_down", "w_up")}
    a = orc.forward(base, w_id, x)
    b = orc.forward(std, w_std, x)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["out"], b["out"])       # bit-exact in fp64
    assert np.array_equal(a["gate"], b["gate"])


def test_identity_projection_latent_equals_input(orc):
    spec = workload("tiny_identity").spec
    w, x = _inputs(spec, 8)
    r = orc.forward(spec, w, x, want_latent=True)
    assert np.array_equal(r["latent"], x.astype(np.float64))


# --------------------------------------------------------------------------
# brute force: every expert evaluated, rank-count selection, dense gate mix

SMALL_SPECS = [
    workload("tiny").spec,
    workload("tiny").spec.replace(gating="softmax_all"),
    workload("tiny").spec.replace(gating="sigmoid_topk_norm", router_on_latent=True),
    LayerSpec(d=48, l=16, m=24, n_experts=7, top_k=3, gating="softmax_all", act_dtype="bf16",
              expert_dtype="bf16", has_router_bias=True),
    LayerSpec(d=32, l=32, m=8, n_experts=5, top_k=5, gating="softmax_topk", act_dtype="f32",
              expert_dtype="f32", has_projections=False),
    LayerSpec(d=64, l=32, m=16, n_experts=9, top_k=2, gating="sigmoid_topk_norm",
              act_dtype="bf16", expert_dtype="fp8_e4m3_rowscale"),
]


@pytest.mark.parametrize("spec", SMALL_SPECS, ids=lambda s: "N%dK%d_%s_%s" % (
    s.n_experts, s.top_k, s.gating, s.expert_dtype))
def test_sparse_equals_dense_bruteforce_bit_exact(orc, spec):
    w, x = _inputs(spec, 37, seed=3)
    a = orc.forward(spec, w, x)
    b = orc.forward_dense(spec, w, x)
    assert np.array_equal(a["out"], b["out"])
    G = b["gate_dense"]
    for t in range(x.shape[0]):
        chosen = np.flatnonzero(G[t] != 0)
        assert sorted(a["idx"][t].tolist()) == chosen.tolist()
        for j, e in enumerate(a["idx"][t]):
            assert G[t, e] == a["gate"][t, j]


# --------------------------------------------------------------------------
# textbook special case: N = K = 1 is a two-layer Squared-ReLU MLP

@pytest.mark.parametrize("gating", ["softmax_all", "softmax_topk", "sigmoid_topk_norm"])
@pytest.mark.parametrize("edt", ["f32", "bf16", "fp8_e4m3_rowscale"])
def test_single_expert_is_squared_relu_mlp(orc, gating, edt):
    act = "f32" if edt == "f32" else "bf16"
    spec = LayerSpec(d=40, l=24, m=56, n_experts=1, top_k=1, gating=gating, act_dtype=act,
                     expert_dtype=edt)
    w, x = _inputs(spec, 11, seed=5)
    r = orc.forward(spec, w, x)
    X = orc.upcast(x, act)
    Wd, Wu = _f64(orc, spec, w, "w_down"), _f64(orc, spec, w, "w_up")
    W1 = _f64(orc, spec, w, "w1")[0]
    W2 = _f64(orc, spec, w, "w2")[0]
    U = X @ Wd.T
    H = np.maximum(U @ W1.T, 0.0) ** 2
    ref = (H @ W2.T) @ Wu.T
    assert np.allclose(r["gate"], 1.0, rtol=0, atol=1e-15)
    assert np.all(r["idx"] == 0)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


# --------------------------------------------------------------------------
# textbook special case: K = N with softmax gating is a dense softmax mixture

@pytest.mark.parametrize("gating", ["softmax_all", "softmax_topk"])
def test_all_experts_softmax_is_dense_softmax_mixture(orc, gating):
    spec = LayerSpec(d=32, l=16, m=20, n_experts=6, top_k=6, gating=gating, act_dtype="f32",
                     expert_dtype="f32", router_on_latent=False)
    w, x = _inputs(spec, 9, seed=7)
    r = orc.forward(spec, w, x)
    X = orc.upcast(x, "f32")
    U = X @ _f64(orc, spec, w, "w_down").T
    Z = X @ _f64(orc, spec, w, "w_router").T
    P = softmax(Z, axis=1)
    W1, W2 = _f64(orc, spec, w, "w1"), _f64(orc, spec, w, "w2")
    V = sum(P[:, [e]] * ((np.maximum(U @ W1[e].T, 0) ** 2) @ W2[e].T) for e in range(6))
    ref = V @ _f64(orc, spec, w, "w_up").T
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    # gates in selection order equal the softmax probabilities of those experts
    for t in range(9):
        np.testing.assert_allclose(r["gate"][t], P[t, r["idx"][t]], rtol=1e-13)


def test_sigmoid_gates_all_experts(orc):
    spec = LayerSpec(d=32, l=16, m=8, n_experts=5, top_k=5, gating="sigmoid_topk_norm",
                     act_dtype="f32", expert_dtype="f32")
    w, x = _inputs(spec, 6, seed=8)
    r = orc.forward(spec, w, x, want_logits=True)
    S = expit(r["logits"])
    for t in range(6):
        np.testing.assert_allclose(r["gate"][t], S[t, r["idx"][t]] / S[t].sum(), rtol=1e-13)


# --------------------------------------------------------------------------
# routing invariants

@pytest.mark.parametrize("spec", SMALL_SPECS[:4], ids=str)
def test_topk_selection_invariants(orc, spec):
    w, x = _inputs(spec, 50, seed=11)
    r = orc.forward(spec, w, x, want_logits=True)
    Z, idx, K, N = r["logits"], r["idx"], spec.top_k, spec.n_experts
    for t in range(x.shape[0]):
        ids = idx[t]
        assert len(set(ids.tolist())) == K and ids.min() >= 0 and ids.max() < N
        sel = Z[t, ids]
        rest = np.delete(Z[t], ids)
        if rest.size:
            assert sel.min() >= rest.max()
            srt = np.sort(Z[t])[::-1]
            assert r["margin"][t] == srt[K - 1] - srt[K]
        assert np.all(np.diff(sel) <= 0)  # selection order: descending score
    counts = orc.expert_counts(idx, N)
    assert counts.sum() == x.shape[0] * K


def test_router_bias_is_added_to_logits(orc):
    spec = LayerSpec(d=32, l=16, m=8, n_experts=12, top_k=3, act_dtype="f32", expert_dtype="f32",
                     has_router_bias=True)
    w, x = _inputs(spec, 10, seed=2)
    r1 = orc.forward(spec, w, x, want_logits=True)
    w0 = dict(w, router_bias=np.zeros_like(w["router_bias"]))
    r0 = orc.forward(spec, w0, x, want_logits=True)
    np.testing.assert_allclose(r1["logits"] - r0["logits"],
                               np.broadcast_to(w["router_bias"].astype(np.float64), r0["logits"].shape),
                               rtol=0, atol=1e-15)


def test_ties_break_toward_lower_expert_id(orc):
    spec = LayerSpec(d=16, l=8, m=8, n_experts=10, top_k=3, gating="softmax_all",
                     act_dtype="f32", expert_dtype="f32")
    w, x = _inputs(spec, 4, seed=4)
    x = np.abs(x)                                   # positive tokens
    wr = np.zeros((10, 16), np.float32)
    wr[[2, 5, 7, 8], :] = 0.25                       # four experts tie for the top logit
    r = orc.forward(spec, dict(w, w_router=wr), x)
    for t in range(4):
        assert r["idx"][t].tolist() == [2, 5, 7]
        assert r["margin"][t] == 0.0
    d = orc.forward_dense(spec, dict(w, w_router=wr), x)
    assert np.array_equal(r["out"], d["out"])


def test_router_on_x_ignores_down_projection(orc):
    spec = workload("tiny").spec
    w, x = _inputs(spec, 20, seed=9)
    a = orc.forward(spec, w, x)
    w2 = dict(w, w_down=(w["w_down"] * np.float32(-3.0)))
    b = orc.forward(spec, w2, x)
    assert np.array_equal(a["idx"], b["idx"])
    assert not np.allclose(a["out"], b["out"])


def test_latent_router_with_identity_down_equals_router_on_x(orc):
    spec = workload("tiny_identity").spec
    lat = spec.replace(router_on_latent=True)
    w, x = _inputs(spec, 30, seed=6)
    a = orc.forward(spec, w, x)
    b = orc.forward(lat, w, x)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("spec", SMALL_SPECS[:4], ids=str)
def test_gate_sums(orc, spec):
    w, x = _inputs(spec, 25, seed=12)
    r = orc.forward(spec, w, x, want_logits=True)
    s = r["gate"].sum(axis=1)
    if spec.gating == "softmax_all":
        P = softmax(r["logits"], axis=1)
        Psel = np.take_along_axis(P, r["idx"].astype(np.int64), axis=1)
        np.testing.assert_allclose(r["gate"], Psel, rtol=1e-12)
        assert np.all(s <= 1.0 + 1e-15)
        renorm = orc.forward(spec.replace(gating="softmax_topk"), w, x)
        np.testing.assert_allclose(r["gate"], renorm["gate"] * s[:, None], rtol=1e-12)
    else:
        np.testing.assert_allclose(s, 1.0, rtol=1e-14)


def test_forced_selection_matches_own_selection(orc):
    spec = workload("tiny").spec
    w, x = _inputs(spec, 16, seed=1)
    a = orc.forward(spec, w, x)
    b = orc.forward(spec, w, x, forced=a["idx"][:, ::-1].copy())
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(b["gate"], a["gate"][:, ::-1])


def test_token_subset_matches_full_evaluation(orc):
    spec = workload("tiny").spec
    w, x = _inputs(spec, 64)
    a = orc.forward(spec, w, x)
    tok = [63, 0, 17, 17, 40]
    b = orc.forward(spec, w, x, tokens=tok)
    assert np.array_equal(b["out"], a["out"][tok])
    assert np.array_equal(b["idx"], a["idx"][tok])


def test_rejects_invalid_configs(orc):
    spec = workload("tiny").spec
    w, x = _inputs(spec, 4)
    with pytest.raises(ValueError):
        orc.forward(spec.replace(top_k=17), w, x)
    with pytest.raises(ValueError):
        orc.forward(spec.replace(has_projections=False), w, x)   # l != d


# --------------------------------------------------------------------------
# storage formats

def test_e4m3_decoder_special_values(orc):
    assert orc.e4m3_to_f64(0x00) == 0.0
    assert math.copysign(1.0, orc.e4m3_to_f64(0x80)) == -1.0
    assert orc.e4m3_to_f64(0x01) == 2.0 ** -9        # smallest subnormal
    assert orc.e4m3_to_f64(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert orc.e4m3_to_f64(0x08) == 2.0 ** -6        # smallest normal
    assert orc.e4m3_to_f64(0x38) == 1.0
    assert orc.e4m3_to_f64(0x7E) == 448.0            # largest finite
    assert orc.e4m3_to_f64(0xFE) == -448.0
    assert math.isnan(orc.e4m3_to_f64(0x7F)) and math.isnan(orc.e4m3_to_f64(0xFF))
    vals = [orc.e4m3_to_f64(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))  # codes are monotonic
    assert len(set(vals)) == 0x7F


def test_e4m3_encoder_round_trips_every_finite_code(orc, syn):
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        v = orc.e4m3_to_f64(c)
        if c == 0x80:
            continue                                    # -0 encodes as +0 magnitude
        assert syn.f64_to_e4m3(v) == c, hex(c)
    # midpoints round to even, values past 448 saturate
    assert syn.f64_to_e4m3(1.0625) == 0x38              # 1 + 1/16: tie -> even (1.0)
    assert syn.f64_to_e4m3(1.1875) == 0x3A              # 1.125/1.25 tie -> even mantissa 2
    assert syn.f64_to_e4m3(500.0) == 0x7E and syn.f64_to_e4m3(-1e9) == 0xFE
    assert syn.f64_to_e4m3(2.0 ** -10) == 0x00          # half the smallest subnormal -> even 0
    assert syn.f64_to_e4m3(3 * 2.0 ** -10) == 0x02      # 1.5 steps -> 2


def test_fp8_row_quantiser_error_bound(orc, syn):
    rows, cols, std = 64, 512, 0.05
    q, s = syn.normal_fp8_rows(3, 9, rows, cols, std)
    w = syn.normal(3, 9, (rows, cols), std, "f64")
    deq = orc.upcast(q, "fp8_e4m3_rowscale", s)
    for r in range(rows):
        a = np.abs(w[r] / s[r])
        err = np.abs(deq[r] - w[r])
        normal = a >= 2.0 ** -6
        assert np.all(err[normal] <= 2.0 ** -4 * np.abs(w[r][normal]) * (1 + 1e-12))
        assert np.all(err[~normal] <= s[r] * 2.0 ** -10 * (1 + 1e-12))
        k = np.argmax(np.abs(w[r]))
        assert abs(orc.e4m3_to_f64(q[r, k])) == 448.0   # row amax maps to +-448
        assert np.float32(np.abs(w[r]).max() / 448.0) == s[r]


def test_bf16_generator_rounds_to_nearest_even(orc, syn):
    w64 = syn.normal(5, 2, (20000,), 1.0, "f64")
    b = syn.normal(5, 2, (20000,), 1.0, "bf16")
    v = orc.upcast(b, "bf16")
    up = orc.upcast((b.astype(np.uint32) + 1).astype(np.uint16), "bf16")
    dn = orc.upcast((b.astype(np.uint32) - 1).astype(np.uint16), "bf16")
    # v is at least as close as either neighbour in the bf16 grid
    assert np.all(np.abs(v - w64) <= np.abs(up - w64))
    assert np.all(np.abs(v - w64) <= np.abs(dn - w64))
    # exact ties go to the even code
    assert syn.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    assert syn.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82


def test_latent_router_reads_unrounded_latent(orc):
    """Closed form: l = d = 2, W_down = [[1, 2^-10], [1, 0]] and x = (1, 1) give
    u = (1 + 2^-10, 1), which bf16 cannot hold (it would round u_0 to 1).
    Router rows e0 = (0, 1) and e1 = (1, 0) on u: z = (1, 1 + 2^-10) exactly,
    so with K = 1 expert 1 wins by a margin of exactly 2^-10.  An oracle that
    rounded u to bf16 before routing would see a tie and pick expert 0."""
    one, tiny = 0x3F80, 0x3A80                    # bf16 bits of 1 and 2^-10
    spec = LayerSpec(d=2, l=2, m=1, n_experts=2, top_k=1, gating="softmax_topk",
                     act_dtype="bf16", expert_dtype="bf16", router_on_latent=True)
    b = lambda a: np.array(a, np.uint16)
    w = {"w_down": b([[one, tiny], [one, 0]]), "w_router": b([[0, one], [one, 0]]),
         "w1": b([[[one, 0]], [[one, 0]]]), "w2": b([[[one], [0]], [[one], [0]]]),
         "w_up": b([[one, 0], [0, one]])}
    x = b([[one, one]])
    assert orc.bf16_to_f64(tiny) == 2.0 ** -10
    for r in (orc.forward(spec, w, x, want_logits=True, want_latent=True),
              orc.route(spec, w, x, want_logits=True)):
        assert r["logits"].tolist() == [[1.0, 1.0 + 2.0 ** -10]]
        assert r["idx"].tolist() == [[1]]
        assert r["margin"].tolist() == [2.0 ** -10]
    f = orc.forward(spec, w, x, want_latent=True)
    assert f["latent"].tolist() == [[1.0 + 2.0 ** -10, 1.0]]
    # expert 1 (gate 1): y = W2_1 (max(0, W1_1 u))^2 = ((1 + 2^-10)^2, 0), out = y
    assert f["out"].tolist() == [[(1.0 + 2.0 ** -10) ** 2, 0.0]]


ROUTE_SPECS = SMALL_SPECS + [
    LayerSpec(d=96, l=48, m=16, n_experts=40, top_k=6, gating="sigmoid_topk_norm",
              act_dtype="bf16", expert_dtype="bf16", router_on_latent=True),
    LayerSpec(d=64, l=64, m=16, n_experts=130, top_k=9, gating="softmax_all", act_dtype="bf16",
              expert_dtype="bf16", has_projections=False, has_router_bias=True),
]


@pytest.mark.parametrize("spec", ROUTE_SPECS, ids=lambda s: "N%dK%d_%s_lat%d" % (
    s.n_experts, s.top_k, s.act_dtype, s.router_on_latent))
def test_route_equals_forward_routing(orc, spec):
    """The routing-only entry returns the ids, margins and logits that the
    full evaluation takes, bit for bit, for every token."""
    w, x = _inputs(spec, 37, seed=21)
    a = orc.forward(spec, w, x, want_logits=True)
    b = orc.route(spec, w, x, want_logits=True)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["margin"], b["margin"])
    assert np.array_equal(a["logits"], b["logits"])


def test_route_crafted_ties_lower_id_wins(orc):
    """Exact ties placed across the K-th position: the lower ids are taken."""
    spec = LayerSpec(d=16, l=8, m=8, n_experts=70, top_k=4, gating="softmax_all",
                     act_dtype="f32", expert_dtype="f32")
    w, _ = _inputs(spec, 1, seed=4)
    wr = np.zeros((70, 16), np.float32)
    wr[9, 0] = 3.0                       # a unique leader on token-column 0
    wr[[66, 2, 64, 5, 40], 0] = 2.0      # five tied for the next places
    wr[[1, 3], 1] = 1.0                  # token-column 1: two tied above zeros
    x = np.zeros((3, 16), np.float32)
    x[0, 0] = 1.0                        # leader + ties: {9} + lowest three of the five
    x[1, 1] = 1.0                        # two, then the lowest two of 68 zeros
    r = orc.route(spec, dict(w, w_router=wr), x)
    assert sorted(r["idx"][0].tolist()) == [2, 5, 9, 40]
    assert sorted(r["idx"][1].tolist()) == [0, 1, 2, 3]
    assert r["idx"][2].tolist() == [0, 1, 2, 3]      # all-zero logits: ids in order
    assert r["margin"].tolist() == [0.0, 0.0, 0.0]
