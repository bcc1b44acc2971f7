"""fp64 CPU oracle of the LatentMoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links
or calls it, and the two share no code; the seeded input generator
(``synth``) is the only module both sides use.

The layer (LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in
Mixture of Experts, §3 Eq. (1)/(2), routed and shared terms) is evaluated token by
token in plain C (``latentmoe_oracle.c``), in fp64, with OpenMP over tokens.
The closed forms of the paper's cost model are in ``cost_model.py``.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(identity reduction, dense brute force, textbook special cases, invariants,
the cost model's printed values).  The layer's output values at the large
workload sizes have no printed worked example on the pages; they rest on the
definition plus those pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "latentmoe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblatentmoe_oracle.so")
_lock = threading.Lock()
_lib = None

_DT = {"f32": 0, "bf16": 1, "fp8_e4m3_rowscale": 2, "mxfp4_e2m1": 3}
_GATE = {"softmax_all": 0, "softmax_topk": 1, "sigmoid_topk_norm": 2}
_ACT = {"sqrelu": 0, "swiglu": 1}


class _Layer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("l", ctypes.c_int64), ("m", ctypes.c_int64),
                ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("router_on_latent", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("has_projections", ctypes.c_int32), ("has_router_bias", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
                ("n_shared", ctypes.c_int64), ("m_shared", ctypes.c_int64),
                ("activation", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("w_down", ctypes.c_void_p), ("w_router", ctypes.c_void_p),
                ("router_bias", ctypes.c_void_p), ("w1", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w1_scale", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_shared1", ctypes.c_void_p), ("w_shared2", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_gate_scale", ctypes.c_void_p),
                ("w_shared_gate", ctypes.c_void_p), ("w1_mx", ctypes.c_void_p),
                ("w2_mx", ctypes.c_void_p), ("w_gate_mx", ctypes.c_void_p)]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                               "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i64 = ctypes.c_void_p, ctypes.c_int64
            lib.orc_forward.argtypes = [ctypes.POINTER(_Layer), ctypes.POINTER(_Weights), vp, vp,
                                        i64, vp, vp, vp, vp, vp, vp, vp]
            lib.orc_forward.restype = ctypes.c_int
            lib.orc_route.argtypes = [ctypes.POINTER(_Layer), ctypes.POINTER(_Weights), vp, i64,
                                      vp, vp, vp]
            lib.orc_route.restype = ctypes.c_int
            lib.orc_forward_dense.argtypes = [ctypes.POINTER(_Layer), ctypes.POINTER(_Weights),
                                              vp, vp, i64, vp, vp]
            lib.orc_forward_dense.restype = ctypes.c_int
            lib.orc_set_threads.argtypes = [ctypes.c_int]
            lib.orc_set_threads.restype = None
            lib.orc_max_threads.argtypes = []
            lib.orc_max_threads.restype = ctypes.c_int
            lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
            lib.orc_bf16_to_f64.restype = ctypes.c_double
            lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
            lib.orc_e4m3_to_f64.restype = ctypes.c_double
            lib.orc_e2m1_to_f64.argtypes = [ctypes.c_uint8]
            lib.orc_e2m1_to_f64.restype = ctypes.c_double
            lib.orc_e8m0_to_f64.argtypes = [ctypes.c_uint8]
            lib.orc_e8m0_to_f64.restype = ctypes.c_double
            _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _layer(spec) -> _Layer:
    return _Layer(spec.d, spec.l, spec.m, spec.n_experts, spec.top_k,
                  int(spec.router_on_latent), _GATE[spec.gating], int(spec.has_projections),
                  int(spec.has_router_bias), _DT[spec.act_dtype], _DT[spec.expert_dtype],
                  spec.n_shared, spec.m_shared, _ACT[spec.activation])


def _weights(w: dict):
    keep = {k: np.ascontiguousarray(v) for k, v in w.items()}
    cw = _Weights(*(_p(keep.get(k)) for k in ("w_down", "w_router", "router_bias", "w1", "w2",
                                               "w1_scale", "w2_scale", "w_up",
                                               "w_shared1", "w_shared2", "w_gate",
                                               "w_gate_scale", "w_shared_gate", "w1_mx",
                                               "w2_mx", "w_gate_mx")))
    return cw, keep


def forward(spec, weights: dict, x: np.ndarray, tokens=None, forced=None,
            want_logits: bool = False, want_latent: bool = False) -> dict:
    """Evaluate the layer for `tokens` (default: every row of x).

    Returns out [n][d], idx [n][K] (z desc, id asc), gate [n][K],
    margin [n] (z_(K) - z_(K+1), +inf for K == N), and optionally logits
    [n][N] and latent [n][l], all float64 / int32.
    """
    lib = _load()
    x = np.ascontiguousarray(x)
    n = x.shape[0] if tokens is None else len(tokens)
    tok = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, np.int64))
    K, N = spec.top_k, spec.n_experts
    f = None
    if forced is not None:
        f = np.ascontiguousarray(np.asarray(forced, np.int32).reshape(n, K))
    res = {"out": np.empty((n, spec.d)), "idx": np.empty((n, K), np.int32),
           "gate": np.empty((n, K)), "margin": np.empty((n,))}
    res["logits"] = np.empty((n, N)) if want_logits else None
    res["latent"] = np.empty((n, spec.l)) if want_latent else None
    L = _layer(spec)
    cw, keep = _weights(weights)
    rc = lib.orc_forward(ctypes.byref(L), ctypes.byref(cw), _p(x), _p(tok), n, _p(f),
                         _p(res["out"]), _p(res["idx"]), _p(res["gate"]), _p(res["margin"]),
                         _p(res["logits"]), _p(res["latent"]))
    del keep
    if rc != 0:
        raise ValueError("oracle rejected the layer configuration or inputs")
    return res


def route(spec, weights: dict, x: np.ndarray, want_logits: bool = False) -> dict:
    """Routing alone for every row of x: idx [T][K] (z desc, id asc), margin
    [T] (z_(K) - z_(K+1)) and optionally the fp64 logits [T][N] (with the
    router bias); no expert is evaluated."""
    lib = _load()
    x = np.ascontiguousarray(x)
    n = x.shape[0]
    K, N = spec.top_k, spec.n_experts
    res = {"idx": np.empty((n, K), np.int32), "margin": np.empty((n,))}
    res["logits"] = np.empty((n, N)) if want_logits else None
    L = _layer(spec)
    cw, keep = _weights(weights)
    rc = lib.orc_route(ctypes.byref(L), ctypes.byref(cw), _p(x), n, _p(res["idx"]),
                       _p(res["margin"]), _p(res["logits"]))
    del keep
    if rc != 0:
        raise ValueError("oracle rejected the layer configuration or inputs")
    return res


def forward_dense(spec, weights: dict, x: np.ndarray, tokens=None) -> dict:
    """Brute-force reference: all experts evaluated, dense masked gate mix."""
    lib = _load()
    x = np.ascontiguousarray(x)
    n = x.shape[0] if tokens is None else len(tokens)
    tok = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, np.int64))
    out = np.empty((n, spec.d))
    G = np.empty((n, spec.n_experts))
    L = _layer(spec)
    cw, keep = _weights(weights)
    rc = lib.orc_forward_dense(ctypes.byref(L), ctypes.byref(cw), _p(x), _p(tok), n, _p(out), _p(G))
    del keep
    if rc != 0:
        raise ValueError("oracle rejected the layer configuration or inputs")
    return {"out": out, "gate_dense": G}


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP token loops."""
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    """Threads the next oracle call will use."""
    return int(_load().orc_max_threads())


def bf16_to_f64(bits: int) -> float:
    return float(_load().orc_bf16_to_f64(int(bits)))


def e4m3_to_f64(code: int) -> float:
    return float(_load().orc_e4m3_to_f64(int(code)))


def e2m1_to_f64(code: int) -> float:
    return float(_load().orc_e2m1_to_f64(int(code)))


def e8m0_to_f64(e: int) -> float:
    return float(_load().orc_e8m0_to_f64(int(e)))


def upcast(a: np.ndarray, dtype: str, scale=None) -> np.ndarray:
    """Exact fp64 values of a stored tensor (bf16 bits / e4m3 codes x row
    scale / MXFP4 pairs x E8M0 block scales, `scale` then the block scales)."""
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "mxfp4_e2m1":
        codes = np.stack([a & 15, a >> 4], axis=-1).reshape(a.shape[:-1] + (2 * a.shape[-1],))
        vals = np.array([e2m1_to_f64(c) for c in range(16)])[codes]
        sc = np.array([e8m0_to_f64(e) for e in range(256)])[scale]
        return vals * np.repeat(sc, 32, axis=-1)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    table = np.array([e4m3_to_f64(c) for c in range(256)])
    v = table[a]
    if scale is not None:
        v = v * scale.astype(np.float64)[..., None]
    return v


def expert_counts(idx: np.ndarray, n_experts: int) -> np.ndarray:
    return np.bincount(idx.reshape(-1), minlength=n_experts).astype(np.int64)
