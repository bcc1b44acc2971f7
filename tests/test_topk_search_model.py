"""The top-k kernel's selection rule, modelled step for step on the CPU.

The kernel (csrc/routing.hip, topk_gate_kernel) holds expert 64 i + lane as
value i of a lane, maps each logit to a uint32 key whose unsigned order is
the float order (+0 == -0), and finds the K-th largest key tau bit by bit
from the top: tau is the largest v with #{keys >= v} >= K, the search
stopping early when a candidate has exactly K keys at or above it.  The set
is every key above tau and, of the keys equal to tau, the lowest ids; each
member is written at its rank under (key desc, id asc).

This model follows those steps over the same [value index][lane] layout and
must equal the top-K set of LatentMoE §3 (text after Eq. (1)) with ties to
the lower expert id, in (logit desc, id asc) order: a sort, checked here on
random and tie-heavy logits.  It pins the algorithm; the GPU parity tests
pin the kernel.
"""
from __future__ import annotations

import numpy as np


def _order_key(z: np.float32) -> int:
    z = np.float32(z)
    if z == 0:
        z = np.float32(0.0)
    u = int(np.array([z], np.float32).view(np.uint32)[0])
    return (~u) & 0xFFFFFFFF if u & 0x80000000 else u | 0x80000000


def _kernel_model(z: np.ndarray, K: int) -> list[int]:
    N = len(z)
    npl = (N + 63) // 64
    key = np.zeros((npl, 64), np.uint64)          # padding lanes: key 0, never selected
    for e in range(N):
        key[e // 64, e % 64] = _order_key(z[e])

    def count_ge(v: int) -> int:                  # sum over i of popcount(ballot(key[i] >= v))
        return int((key >= v).sum())

    tau, exact = 0, False
    for b in range(31, -1, -1):
        cand = tau | (1 << b)
        c = count_ge(cand)
        if c >= K:
            tau = cand
            if c == K:
                exact = True
                break
    if exact:
        sel = key >= tau
    else:
        sel = np.zeros_like(key, bool)
        r = K - (0 if tau == 0xFFFFFFFF else count_ge(tau + 1))
        for i in range(npl):
            eq = key[i] == tau
            below = np.cumsum(eq) - eq            # mbcnt of the ballot: equal keys on lower lanes
            sel[i] = (key[i] > tau) | (eq & (below < r))
            r -= int(eq.sum())
    ids = [i * 64 + l for i in range(npl) for l in range(64) if sel[i, l]]   # compaction order
    assert len(ids) == K
    comp = [(int(key[e // 64, e % 64]) << 32) | (0xFFFFFFFF - e) for e in ids]
    out = [-1] * K
    for e, me in zip(ids, comp):
        out[sum(c > me for c in comp)] = e        # rank under (key desc, id asc)
    return out


def _sorted_top_k(z: np.ndarray, K: int) -> list[int]:
    return sorted(range(len(z)), key=lambda e: (-float(z[e]), e))[:K]


def test_search_model_equals_sorted_top_k():
    rng = np.random.default_rng(7)
    for trial in range(600):
        N = int(rng.integers(1, 300))
        K = int(rng.integers(1, min(N, 64) + 1))
        kind = trial % 4
        if kind == 0:
            z = rng.standard_normal(N).astype(np.float32)
        elif kind == 1:
            z = rng.integers(-2, 3, N).astype(np.float32)          # many exact ties
        elif kind == 2:
            z = np.where(rng.random(N) < 0.5, 0.0, -0.0).astype(np.float32)
            z[rng.random(N) < 0.1] = 1.0                            # +0 and -0 tie
        else:
            z = (rng.standard_normal(N) * 1e-30).astype(np.float32)  # tiny, subnormal-ish
            z[rng.random(N) < 0.05] = -np.inf
        assert _kernel_model(z, K) == _sorted_top_k(z, K), (N, K, kind)


def test_search_model_full_width_and_all_equal():
    # K = N (every key taken), and every logit equal (the K lowest ids)
    for N, K in [(64, 64), (2048, 64), (512, 22), (896, 16)]:
        z = np.zeros(N, np.float32)
        assert _kernel_model(z, K) == list(range(K))
        z = np.arange(N, dtype=np.float32)
        assert _kernel_model(z, K) == list(range(N - 1, N - 1 - K, -1))
