"""The oracle's cost model against the values the paper prints (CPU only).

Printed values live in tests/golden/paper_printed_values.json, each with the
section of "LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in
Mixture of Experts" it comes from.
"""
import json
import math
import os

import pytest

from oracle import cost_model as cm
from synth import workload

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "paper_printed_values.json")))
EX = GOLD["running_example"]


def test_compute_bound_threshold_is_1250():
    assert cm.compute_bound_threshold(EX["F_flops"], EX["bw_hbm"]) == \
        GOLD["compute_bound_threshold"]["value"]


def test_min_tokens_per_expert_is_1418():
    thr = GOLD["compute_bound_threshold"]["value"]
    d, m = EX["d"], EX["m"]
    root = cm.min_t_exp(d, m, thr)
    assert math.floor(root) == GOLD["min_t_exp"]["value"]
    assert abs(root - 1418.807) < 1e-3
    # the printed integer is the truncated root: 1418 tokens fall just short
    assert cm.intensity(1418, d, m) < thr <= cm.intensity(1419, d, m)
    # with FP4 counted as half a byte the threshold would be far lower
    assert 433 < cm.min_t_exp(d, m, thr, bytes_per_elem=0.5) < 435


def test_intensity_form_matches_flops_over_traffic():
    d, m = EX["d"], EX["m"]
    for t in (1, 32, 704, 5000):
        assert cm.intensity(t, d, m) == pytest.approx(2 * t * d * m / (d * m + t * (d + m)),
                                                      rel=1e-15)
    # two experts per GPU leave the ratio unchanged (2 C / 2 M)
    t = 100
    assert (2 * cm.expert_flops(t, d, m)) / (2 * cm.expert_traffic(t, d, m)) == \
        pytest.approx(cm.intensity(t, d, m), rel=1e-15)


def test_communication_model():
    N, EP, d, m = EX["N"], EX["EP"], EX["d"], EX["m"]
    assert N // EP == GOLD["experts_per_gpu"]["value"]
    t = 77.0
    assert cm.m_comm(N, EP, t, d) == GOLD["m_comm_factor"]["value"] * t * d
    assert cm.c_comp(N, EP, t, d, m) == GOLD["c_comp_factor"]["value"] * t * d * m
    r = cm.comm_compute_ratio(EX["F_flops"], m, EX["bw_nvl"])
    assert round(r) == GOLD["comm_compute_ratio"]["value"]
    assert r == pytest.approx(9.042, abs=1e-3)
    # the ratio is independent of t_exp and d
    tc = cm.m_comm(N, EP, t, d) / EX["bw_nvl"]
    tp = cm.c_comp(N, EP, t, d, m) / EX["F_flops"]
    assert tc / tp == pytest.approx(r, rel=1e-12)


def test_combinatorial_diversity_inequality():
    a = GOLD["alpha_adopted"]["value"]
    N, K = EX["N"], EX["K"]
    lhs = cm.log10_binom(a * N, a * K)
    rhs = a * cm.log10_binom(N, K)
    assert lhs >= rhs
    assert lhs == pytest.approx(50.85, abs=0.01) and rhs == pytest.approx(48.62, abs=0.01)
    assert cm.log10_binom(5, 2) == pytest.approx(1.0)          # C(5,2) = 10


def test_iso_cost_of_latent_variant():
    """l-MoE_acc keeps expert weight bytes and dispatch volume per token equal
    to the standard MoE (§3 text after Eq. (2); Table 1)."""
    std = workload("std_decode").spec
    lat = workload("latent_decode").spec
    a = std.d // lat.l
    assert lat.n_experts == a * std.n_experts and lat.top_k == a * std.top_k
    assert std.top_k * 2 * std.d * std.m == lat.top_k * 2 * lat.l * lat.m
    T = 512
    assert cm.a2a_bytes(std, T)["dispatch"] == cm.a2a_bytes(lat, T)["dispatch"]
    eff = cm.table1("eff", 128, 64, 32, 4096, 1024, 1536)
    stdt = cm.table1("standard", 128, 64, 32, 4096, 1024, 1536)
    acc = cm.table1("acc", 128, 64, 32, 4096, 1024, 1536)
    assert stdt["comm_width"] == a * eff["comm_width"] == acc["comm_width"]
    assert stdt["weight_per_expert"] == a * eff["weight_per_expert"] == acc["weight_per_expert"]


def test_t_exp_of_workloads():
    assert cm.t_exp(512, 8, 128) == 32
    assert cm.t_exp(512, 32, 512) == 32
    assert cm.t_exp(16384, 22, 512) == 704
    assert cm.t_exp(4096, 16, 896) == pytest.approx(73.14, abs=0.01)


def test_layer_counters():
    lat = workload("latent_decode").spec
    f = cm.layer_flops(lat, 512)
    assert f["fc1"] == f["fc2"] == 2 * 512 * 32 * 1024 * 1536
    assert f["total"] == pytest.approx(113.8e9, rel=2e-3)
    b = cm.layer_bytes(lat, 512, touched_experts=512)
    assert b["total"] == pytest.approx(3.251e9, rel=2e-3)
    std = workload("std_decode").spec
    assert cm.layer_bytes(std, 512, 128)["total"] == pytest.approx(3.231e9, rel=2e-3)
    assert cm.a2a_bytes(lat, 512)["paper_fp4_bf16"] == 2.5 * 512 * 32 * 1024
