"""Pins of the oracle's MXFP4 expert weights (CPU only).

MXFP4 here is the OCP Microscaling format: FP4 E2M1 elements, one E8M0
power-of-two scale per block of 32 consecutive elements of a weight row,
element 2j in the low nibble of byte j.  The pins tie the oracle's decoder
to the format's published value table, the generator's quantiser to its
rounding bound, and the MXFP4 layer to the bf16 layer holding the same
decoded values (bit-exact), which pins the nibble order and block indexing.
"""
import math

import numpy as np
import pytest

import synth
from synth import LayerSpec, make_tokens, make_weights

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

# OCP MX v1.0, FP4 E2M1: S.EE.M, bias 1, exponent 0 subnormal (0.5 * M)
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_value_table(orc):
    for code in range(16):
        want = E2M1[code & 7] * (-1.0 if code & 8 else 1.0)
        got = orc.e2m1_to_f64(code)
        assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), code


def test_e8m0_scale(orc):
    assert orc.e8m0_to_f64(127) == 1.0
    assert orc.e8m0_to_f64(0) == 2.0 ** -127
    assert orc.e8m0_to_f64(254) == 2.0 ** 127
    assert orc.e8m0_to_f64(120) == 2.0 ** -7
    assert math.isnan(orc.e8m0_to_f64(255))


def _unpack(q, x):
    """test-side decoding of the documented layout (values from the table)"""
    lo, hi = q & 15, q >> 4
    codes = np.empty(q.shape[:-1] + (2 * q.shape[-1],), np.int64)
    codes[..., 0::2], codes[..., 1::2] = lo, hi
    tab = np.array([E2M1[c & 7] * (-1.0 if c & 8 else 1.0) for c in range(16)])
    return tab[codes] * np.repeat(np.ldexp(1.0, x.astype(np.int64) - 127), 32, axis=-1)


def test_quantiser_round_trips_every_code_and_meets_the_rounding_bound(orc):
    # every code at several scales: a block whose largest magnitude is 6 * 2^X
    # keeps the scale X and every code
    for X in (-9, -3, 0, 4):
        codes = np.array([c for c in range(16)] * 2, np.uint8)
        codes[0] = 7                                   # max 6 * 2^X fixes the scale
        v = np.array([E2M1[c & 7] * (-1.0 if c & 8 else 1.0) for c in codes]) * 2.0 ** X
        q, x = synth.mxfp4_quantize(v[None, :])
        assert int(x[0, 0]) == X + 127
        dec = orc.upcast(q, "mxfp4_e2m1", x)[0]
        assert np.array_equal(dec, v)
    # normals: |q - v| is at most half the E2M1 spacing around |v| / 2^X, or
    # the saturation overshoot above 6 * 2^X
    v = synth.normal(3, 55, (64, 256), 0.7, "f64")
    q, x = synth.mxfp4_quantize(v)
    dec = orc.upcast(q, "mxfp4_e2m1", x)
    scale = np.repeat(np.ldexp(1.0, x.astype(np.int64) - 127), 32, axis=-1)
    a = np.abs(v) / scale
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = np.where(a > 6, a - 6, half) * scale
    assert (np.abs(dec - v) <= bound * (1 + 1e-12)).all()
    assert (np.abs(v) / scale).max() < 8          # X = floor(log2 amax) - 2


def _bf16_bits(vals):
    f = vals.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), vals)        # exact in fp32
    b = f.view(np.uint32)
    assert (b & 0xFFFF).max() == 0                            # and in bf16
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("act", ["sqrelu", "swiglu"])
def test_mxfp4_layer_equals_bf16_layer_with_the_decoded_weights(orc, act):
    mx = LayerSpec(d=96, l=64, m=96, n_experts=7, top_k=3, gating="softmax_topk",
                   expert_dtype="mxfp4_e2m1", activation=act)
    bf = mx.replace(expert_dtype="bf16")
    w = make_weights(mx, 8)
    x = make_tokens(mx, 19, 8)
    wb = {k: v for k, v in w.items() if not k.endswith("_mx")}
    for k in ("w1", "w2", "w_gate"):
        if k in w:
            wb[k] = _bf16_bits(_unpack(w[k], w[k + "_mx"]))
    a = orc.forward(mx, w, x)
    b = orc.forward(bf, wb, x)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["out"], b["out"])


def test_mxfp4_sparse_equals_dense_bit_exact(orc):
    spec = LayerSpec(d=64, l=32, m=64, n_experts=9, top_k=2, gating="sigmoid_topk_norm",
                     expert_dtype="mxfp4_e2m1", has_router_bias=True)
    w = make_weights(spec, 2)
    x = make_tokens(spec, 23, 2)
    assert np.array_equal(orc.forward(spec, w, x)["out"], orc.forward_dense(spec, w, x)["out"])


def test_mxfp4_needs_whole_blocks_and_scales(orc):
    spec = LayerSpec(d=64, l=32, m=64, n_experts=4, top_k=2, expert_dtype="mxfp4_e2m1")
    w = make_weights(spec, 1)
    x = make_tokens(spec, 3, 1)
    with pytest.raises(ValueError):
        orc.forward(spec, {k: v for k, v in w.items() if k != "w2_mx"}, x)
    with pytest.raises(ValueError):
        orc.forward(spec.replace(l=48), w, x)
