"""Seeded synthetic inputs for the LatentMoE layer forward.

This package builds INPUTS ONLY (tokens, weights, router bias) from a
counter-based SplitMix64 stream + Box-Muller normals, rounded to the storage
dtype.  It holds none of the layer's arithmetic.  It is the one module that
both the fp64 oracle (``oracle/``) and the GPU library's tests and benchmark
use, so that both sides see bit-identical inputs.

Tensor stream ids: x = 0, W_down = 1, W_router = 2, W1 = 3, W2 = 4, W_up = 5,
router-bias permutation = 6, shared W1 = 7, shared W2 = 8, W_gate = 9,
shared W_gate = 10.  Every weight ~ N(0, 1/fan_in); x ~ N(0, 1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .workloads import LayerSpec, WORKLOADS, workload  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

(TID_X, TID_WDOWN, TID_WROUTER, TID_W1, TID_W2, TID_WUP, TID_BIAS, TID_WS1, TID_WS2, TID_WGATE,
 TID_WSGATE) = range(11)


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP).  sin and cos stay
    separate library calls (no merged sincos), so every value is the same
    whether its Box-Muller partner is computed in the same pass or not."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-builtin-sin", "-fno-builtin-cos", "-fopenmp",
                               "-shared", "-fPIC", "-Wall",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            u64, u32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                      ctypes.c_double, ctypes.c_void_p)
            for name in ("synth_normal_f64", "synth_normal_f32", "synth_normal_bf16"):
                f = getattr(lib, name)
                f.argtypes = [u64, u32, u64, i64, dbl, vp]
                f.restype = None
            lib.synth_normal_fp8_rows.argtypes = [u64, u32, u64, i64, i64, dbl, vp, vp]
            lib.synth_normal_fp8_rows.restype = ctypes.c_int
            lib.synth_zipf_bias.argtypes = [u64, u32, i64, dbl, vp]
            lib.synth_zipf_bias.restype = ctypes.c_int
            lib.synth_permutation.argtypes = [u64, u32, i64, vp]
            lib.synth_permutation.restype = None
            lib.synth_raw_u64.argtypes = [u64, u32, u64]
            lib.synth_raw_u64.restype = u64
            lib.synth_f64_to_bf16.argtypes = [dbl]
            lib.synth_f64_to_bf16.restype = ctypes.c_uint16
            lib.synth_f64_to_e4m3.argtypes = [dbl]
            lib.synth_f64_to_e4m3.restype = ctypes.c_uint8
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def normal(seed: int, tid: int, shape, std: float, dtype: str, offset: int = 0) -> np.ndarray:
    """Normals N(0, std^2) for elements offset .. offset+prod(shape) of stream tid.

    dtype: 'f64' -> float64, 'f32' -> float32, 'bf16' -> uint16 bit patterns.
    """
    lib = _load()
    n = int(np.prod(shape))
    if dtype == "f64":
        out = np.empty(shape, np.float64)
        lib.synth_normal_f64(seed, tid, offset, n, std, _ptr(out))
    elif dtype == "f32":
        out = np.empty(shape, np.float32)
        lib.synth_normal_f32(seed, tid, offset, n, std, _ptr(out))
    elif dtype == "bf16":
        out = np.empty(shape, np.uint16)
        lib.synth_normal_bf16(seed, tid, offset, n, std, _ptr(out))
    else:
        raise ValueError("dtype must be f64, f32 or bf16, got %r" % dtype)
    return out


def normal_fp8_rows(seed: int, tid: int, rows: int, cols: int, std: float, offset: int = 0):
    """rows x cols normals quantised per row to OCP E4M3 bytes + fp32 row scales."""
    lib = _load()
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows,), np.float32)
    if lib.synth_normal_fp8_rows(seed, tid, offset, rows, cols, std, _ptr(q), _ptr(s)) != 0:
        raise MemoryError("synth: row buffer allocation failed")
    return q, s


# Thresholds between neighbouring E2M1 magnitudes (0, 0.5, 1, 1.5, 2, 3, 4,
# 6: codes 0..7, codes 8..15 their negatives).  A magnitude exactly at a
# midpoint takes the even code: upwards at 0.75, 1.75 and 3.5 (codes 2, 4,
# 6), downwards at 0.25, 1.25, 2.5 and 5 (codes 0, 2, 4, 6).
_E2M1_UP = (0.75, 1.75, 3.5)
_E2M1_DOWN = (0.25, 1.25, 2.5, 5.0)


def mxfp4_quantize(v: np.ndarray, chunk_rows: int = 4096):
    """OCP MX quantisation of v [rows][cols] (cols a multiple of 32) to FP4
    E2M1 with one E8M0 scale per 32 consecutive elements of a row.

    Per block: X = floor(log2(max |v|)) - 2 (2 = the largest E2M1 exponent),
    clamped to the E8M0 range [-127, 127] (all-zero blocks: -127); elements
    v / 2^X rounded to the nearest E2M1 value, ties to the even code,
    magnitudes above 6 saturated to 6.  Returns (packed [rows][cols/2]
    uint8, element 2j in the low nibble of byte j; scales [rows][cols/32]
    uint8, the biased exponent X + 127).  Rows are processed in chunks.
    """
    v = np.asarray(v, np.float64)
    rows, cols = v.shape
    if cols % 32:
        raise ValueError("MXFP4 rows must hold whole blocks of 32")
    packed = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    for r0 in range(0, rows, chunk_rows):
        blk = v[r0:r0 + chunk_rows].reshape(-1, cols // 32, 32)
        amax = np.abs(blk).max(axis=2)
        with np.errstate(divide="ignore"):
            X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
        X = np.clip(X, -127, 127)
        y = blk / np.ldexp(1.0, X.astype(np.int64))[..., None]
        a = np.abs(y)
        k = np.zeros(a.shape, np.uint8)      # nearest code; past 6 it stays 7
        for t in _E2M1_UP:
            k += a >= t
        for t in _E2M1_DOWN:
            k += a > t
        code = (k + 8 * ((y < 0) & (k > 0))).astype(np.uint8).reshape(-1, cols)
        packed[r0:r0 + chunk_rows] = code[:, 0::2] | (code[:, 1::2] << 4)
        scales[r0:r0 + chunk_rows] = (X + 127).astype(np.uint8)
    return packed, scales


def normal_mxfp4_rows(seed: int, tid: int, rows: int, cols: int, std: float, offset: int = 0):
    """rows x cols normals quantised to MXFP4 (mxfp4_quantize)."""
    return mxfp4_quantize(normal(seed, tid, (rows, cols), std, "f64", offset))


def f64_to_bf16(v: float) -> int:
    return int(_load().synth_f64_to_bf16(float(v)))


def f64_to_e4m3(v: float) -> int:
    return int(_load().synth_f64_to_e4m3(float(v)))


def permutation(seed: int, tid: int, n: int) -> np.ndarray:
    p = np.empty((n,), np.int32)
    _load().synth_permutation(seed, tid, n, _ptr(p))
    return p


def zipf_bias(seed: int, tid: int, n: int, s: float) -> np.ndarray:
    b = np.empty((n,), np.float32)
    if _load().synth_zipf_bias(seed, tid, n, s, _ptr(b)) != 0:
        raise ValueError("zipf_bias supports 1..4096 experts")
    return b


def make_tokens(spec: LayerSpec, T: int, seed: int = 0) -> np.ndarray:
    """x[T][d] ~ N(0, 1) in the activation dtype (uint16 bits for bf16)."""
    return normal(seed, TID_X, (T, spec.d), 1.0, spec.act_dtype)


def make_weights(spec: LayerSpec, seed: int = 0) -> dict:
    """All layer weights for `spec`, as numpy arrays in their storage dtypes.

    Keys: w_down [l][d], w_up [d][l] (absent without projections; the
    identity matrix when spec.identity_projections), w_router [N][d or l],
    router_bias [N] (fp32, only with spec.has_router_bias), w1 [N][m][l],
    w2 [N][l][m] (+ w1_scale [N][m], w2_scale [N][l] for fp8 experts);
    MXFP4 experts: w1 [N][m][l/2], w2 [N][l][m/2] packed E2M1 pairs with
    E8M0 block scales w1_mx [N][m][l/32], w2_mx [N][l][m/32].
    SwiGLU experts add w_gate [N][m][l] (+ w_gate_scale [N][m]); shared
    experts w_shared1 [S*ms][d], w_shared2 [d][S*ms] and, with SwiGLU,
    w_shared_gate [S*ms][d].
    """
    d, l, m, N = spec.d, spec.l, spec.m, spec.n_experts
    act = spec.act_dtype
    w = {}
    if spec.has_projections:
        if spec.identity_projections:
            if l != d:
                raise ValueError("identity projections need l == d")
            eye = np.eye(d, dtype=np.float64)
            if act == "f32":
                w["w_down"] = eye.astype(np.float32)
            else:
                w["w_down"] = np.where(eye == 1.0, np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
            w["w_up"] = w["w_down"].copy()
        else:
            w["w_down"] = normal(seed, TID_WDOWN, (l, d), d ** -0.5, act)
            w["w_up"] = normal(seed, TID_WUP, (d, l), l ** -0.5, act)
    r_in = l if spec.router_on_latent else d
    w["w_router"] = normal(seed, TID_WROUTER, (N, r_in), r_in ** -0.5, act)
    if spec.has_router_bias:
        w["router_bias"] = zipf_bias(seed, TID_BIAS, N, spec.zipf_s)
    if spec.expert_dtype == "mxfp4_e2m1":
        q1, x1 = normal_mxfp4_rows(seed, TID_W1, N * m, l, l ** -0.5)
        q2, x2 = normal_mxfp4_rows(seed, TID_W2, N * l, m, m ** -0.5)
        w["w1"], w["w1_mx"] = q1.reshape(N, m, l // 2), x1.reshape(N, m, l // 32)
        w["w2"], w["w2_mx"] = q2.reshape(N, l, m // 2), x2.reshape(N, l, m // 32)
        if spec.activation == "swiglu":
            qg, xg = normal_mxfp4_rows(seed, TID_WGATE, N * m, l, l ** -0.5)
            w["w_gate"], w["w_gate_mx"] = qg.reshape(N, m, l // 2), xg.reshape(N, m, l // 32)
    elif spec.expert_dtype == "fp8_e4m3_rowscale":
        q1, s1 = normal_fp8_rows(seed, TID_W1, N * m, l, l ** -0.5)
        q2, s2 = normal_fp8_rows(seed, TID_W2, N * l, m, m ** -0.5)
        w["w1"], w["w1_scale"] = q1.reshape(N, m, l), s1.reshape(N, m)
        w["w2"], w["w2_scale"] = q2.reshape(N, l, m), s2.reshape(N, l)
        if spec.activation == "swiglu":
            qg, sg = normal_fp8_rows(seed, TID_WGATE, N * m, l, l ** -0.5)
            w["w_gate"], w["w_gate_scale"] = qg.reshape(N, m, l), sg.reshape(N, m)
    else:
        w["w1"] = normal(seed, TID_W1, (N, m, l), l ** -0.5, spec.expert_dtype)
        w["w2"] = normal(seed, TID_W2, (N, l, m), m ** -0.5, spec.expert_dtype)
        if spec.activation == "swiglu":
            w["w_gate"] = normal(seed, TID_WGATE, (N, m, l), l ** -0.5, spec.expert_dtype)
    if spec.n_shared:
        # shared experts, in the activation dtype: w_shared1 [S*ms][d] (expert
        # j's rows j*ms ..), w_shared2 [d][S*ms] (expert j's columns j*ms ..)
        S, ms = spec.n_shared, spec.m_shared
        w["w_shared1"] = normal(seed, TID_WS1, (S * ms, d), d ** -0.5, act)
        w["w_shared2"] = normal(seed, TID_WS2, (d, S * ms), ms ** -0.5, act)
        if spec.activation == "swiglu":
            w["w_shared_gate"] = normal(seed, TID_WSGATE, (S * ms, d), d ** -0.5, act)
    return w
