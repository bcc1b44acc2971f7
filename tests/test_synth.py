"""The seeded input generator: determinism, slicing, distributions (CPU only)."""
import numpy as np

import synth
from synth import workload


def test_streams_are_deterministic_and_sliceable(syn):
    a = syn.normal(0, 3, (1000,), 0.5, "f64")
    b = syn.normal(0, 3, (1000,), 0.5, "f64")
    assert np.array_equal(a, b)
    c = syn.normal(0, 3, (200,), 0.5, "f64", offset=401)
    assert np.array_equal(c, a[401:601])
    assert not np.array_equal(a, syn.normal(1, 3, (1000,), 0.5, "f64"))
    assert not np.array_equal(a, syn.normal(0, 4, (1000,), 0.5, "f64"))


def test_normal_moments(syn):
    a = syn.normal(7, 0, (400000,), 2.0, "f64")
    assert abs(a.mean()) < 0.02 and abs(a.std() - 2.0) < 0.02
    b = syn.normal(7, 0, (400000,), 2.0, "f32")
    assert np.array_equal(b, a.astype(np.float32))


def test_permutation_and_zipf_bias(syn):
    p = syn.permutation(0, 6, 512)
    assert sorted(p.tolist()) == list(range(512))
    b = syn.zipf_bias(0, 6, 512, 1.1)
    np.testing.assert_allclose(b, -1.1 * np.log(p + 1.0), rtol=1e-6)
    assert b.max() == 0.0


def test_layer_weight_shapes():
    spec = workload("tiny").spec
    w = synth.make_weights(spec)
    assert w["w_down"].shape == (64, 256) and w["w_up"].shape == (256, 64)
    assert w["w_router"].shape == (16, 256)
    assert w["w1"].shape == (16, 128, 64) and w["w2"].shape == (16, 64, 128)
    x = synth.make_tokens(spec, 64)
    assert x.shape == (64, 256) and x.dtype == np.float32
    # tokens for a prefix of a longer batch are the same rows
    assert np.array_equal(synth.make_tokens(spec, 10), x[:10])
    s8 = spec.replace(act_dtype="bf16", expert_dtype="fp8_e4m3_rowscale")
    w8 = synth.make_weights(s8)
    assert w8["w1"].dtype == np.uint8 and w8["w1_scale"].shape == (16, 128)
    assert w8["w2_scale"].shape == (16, 64)
