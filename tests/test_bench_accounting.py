"""The benchmark's algorithmic byte and FLOP counts (CPU only).

With every expert touched they must equal the layer's closed forms: weights
of the experts, projections and router read once, x read once, out written
once; FLOPs 2*T*d*l per projection, 2*T*d*N for the router, 4*T*K*l*m for
the experts (6*T*K*l*m with SwiGLU).  The expected totals are written out
from those definitions for the decode, prefill and fp8 shapes.
"""
import numpy as np
import pytest

import bench
from synth import workload


def _all_touched(spec):
    return np.ones(spec.n_experts, np.int64)


# (bytes, FLOPs) written out from the definitions, every expert touched
EXACT = {
    # T 512, d 4096, m 1536, N 128, K 8, no projections, bf16
    "std_decode": (128 * 2 * 4096 * 1536 * 2 + 128 * 4096 * 2 + 2 * 512 * 4096 * 2,
                   2 * 512 * 4096 * 128 + 4 * 512 * 8 * 4096 * 1536),
    # T 512, d 4096, l 1024, m 1536, N 512, K 32, bf16
    "latent_decode": (512 * 2 * 1024 * 1536 * 2 + 512 * 4096 * 2 + 2 * 512 * 4096 * 2
                      + 2 * 1024 * 4096 * 2,
                      2 * 512 * 4096 * 512 + 4 * 512 * 32 * 1024 * 1536 + 4 * 512 * 4096 * 1024),
    # T 16384, d 4096, l 1024, m 2048, N 512, K 22, fp32 router bias, bf16
    "latent_prefill_zipf": (512 * 2 * 1024 * 2048 * 2 + 512 * 4096 * 2 + 2 * 16384 * 4096 * 2
                            + 4 * 512 + 2 * 1024 * 4096 * 2,
                            2 * 16384 * 4096 * 512 + 4 * 16384 * 22 * 1024 * 2048
                            + 4 * 16384 * 4096 * 1024),
    # T 4096, d 7168, l 1792, m 2048, N 896, K 16, fp8 experts + fp32 row scales
    "latent_fp8_sparse": (896 * (2 * 1792 * 2048 + 4 * (2048 + 1792)) + 896 * 7168 * 2
                          + 2 * 4096 * 7168 * 2 + 2 * 1792 * 7168 * 2,
                          2 * 4096 * 7168 * 896 + 4 * 4096 * 16 * 1792 * 2048
                          + 4 * 4096 * 7168 * 1792),
}


@pytest.mark.parametrize("name", list(EXACT))
def test_layer_totals_match_the_closed_forms(name):
    wl = workload(name)
    nbytes, flops = bench.layer_work(wl.spec, wl.T, _all_touched(wl.spec))
    assert (nbytes, flops) == EXACT[name]


def test_closed_forms_round_to_the_printed_totals():
    # 3.231 / 3.251 / 4.58 / 6.77 GB and 103.6 / 113.8 / 3367 / 1225 GFLOP
    got = {k: (round(b / 1e9, 3), round(f / 1e9, 1)) for k, (b, f) in EXACT.items()}
    assert got["std_decode"] == (3.231, 103.6)
    assert got["latent_decode"] == (3.251, 113.8)
    assert got["latent_prefill_zipf"][0] == pytest.approx(4.58, abs=0.01)
    assert round(got["latent_prefill_zipf"][1]) == 3367
    assert got["latent_fp8_sparse"][0] == pytest.approx(6.77, abs=0.005)
    assert round(got["latent_fp8_sparse"][1]) == 1225


def test_expert_stage_bytes_and_flops():
    """An expert launch's algorithmic bytes are the expert weights it must
    read (token rows, H and Y are intermediates); FLOPs 2*T*K*l*m per GEMM."""
    wl = workload("latent_decode")
    s, T = wl.spec, wl.T
    c = _all_touched(s)
    w = 512 * 1024 * 1536 * 2                         # one weight set of all experts
    b1, f1 = bench.expert_kernel_work(s, T, c, "fc1")
    b2, f2 = bench.expert_kernel_work(s, T, c, "fc2")
    bf, ff = bench.expert_kernel_work(s, T, c, "ffn")
    assert b1 == b2 == w and bf == 2 * w
    assert f1 == f2 == 2 * T * 32 * 1024 * 1536 and ff == f1 + f2
    # only experts that received tokens are read
    half = np.arange(s.n_experts) % 2
    assert bench.expert_kernel_work(s, T, half, "ffn")[0] == w
    # SwiGLU: FC1 reads and multiplies twice the rows
    g = s.replace(activation="swiglu")
    b1g, f1g = bench.expert_kernel_work(g, T, c, "fc1")
    assert b1g == 2 * w and f1g == 2 * f1
    # MXFP4: half a byte per weight plus a scale byte per 32
    x = s.replace(expert_dtype="mxfp4_e2m1")
    b1x, _ = bench.expert_kernel_work(x, T, c, "fc1")
    assert b1x == pytest.approx(w / 2 * (0.5 + 1 / 32))
    # fp8 (the 896-expert layer): one byte per weight plus an fp32 scale per row
    f8 = workload("latent_fp8_sparse").spec
    c8 = _all_touched(f8)
    assert bench.expert_kernel_work(f8, 4096, c8, "fc1")[0] == 896 * (2048 * 1792 + 4 * 2048)
    assert bench.expert_kernel_work(f8, 4096, c8, "fc2")[0] == 896 * (1792 * 2048 + 4 * 1792)


def test_shared_experts_add_their_weights_and_flops():
    base, sh = workload("latent_decode").spec, workload("latent_decode_shared").spec
    c = _all_touched(base)
    b0, f0 = bench.layer_work(base, 512, c)
    b1, f1 = bench.layer_work(sh, 512, c)
    assert b1 - b0 == 2 * 4096 * (2 * 1536) * 2         # Ws1 and Ws2, bf16
    assert f1 - f0 == 4 * 512 * 4096 * (2 * 1536)


@pytest.mark.parametrize("name", ["t2_std", "t2_eff_a4", "t2_acc_a4", "latent_swiglu_decode",
                                  "latent_fp8_sparse"])
def test_sweep_summary_bytes_equal_the_bench_definition(name):
    """The alpha-sweep summary recomputes FC1 + FC2's algorithmic bytes
    from a bench line's config and touched-expert count; they equal the
    benchmark's own expert-weight bytes of the two GEMMs."""
    from mixture_experts_layer_32_amd import profiling
    spec = workload(name).spec
    counts = np.zeros(spec.n_experts, np.int64)
    counts[::3] = 5                                    # a third of the experts touched
    touched = int((counts > 0).sum())
    cfg = {"l": spec.l, "m": spec.m, "activation": spec.activation,
           "expert_dtype": spec.expert_dtype}
    want = bench.expert_weight_bytes(spec, counts, "fc1") + bench.expert_weight_bytes(spec, counts, "fc2")
    assert profiling._expert_weight_bytes(cfg, touched) == want
