"""MI355X (gfx950) LatentMoE layer forward -- Python binding of liblatentmoe.so.

The layer (LatentMoE: Toward Optimal Accuracy per FLOP and Parameter in
Mixture of Experts, §3 Eq. (1)/(2), routed and shared experts) runs entirely in the
HIP kernels behind the C ABI declared in ``include/latentmoe.h``.  This module
only marshals arguments: it checks shapes/dtypes of torch tensors, passes
their device pointers, the current HIP stream and a workspace tensor, and
maps status codes to exceptions.  PyTorch is used for device memory and
streams only.  There is no CPU fallback: if the library is missing the
import of ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblatentmoe.so")   # the in-tree build

LMOE_F32, LMOE_BF16, LMOE_FP8_E4M3_ROWSCALE, LMOE_MXFP4_E2M1 = 0, 1, 2, 3
ROUTER_ON_X, ROUTER_ON_LATENT = 0, 1
GATE_SOFTMAX_ALL, GATE_SOFTMAX_TOPK, GATE_SIGMOID_TOPK_NORM = 0, 1, 2
ACT_SQRELU, ACT_SWIGLU = 0, 1
_ACT = {"sqrelu": ACT_SQRELU, "swiglu": ACT_SWIGLU}
# expert-FFN kernel choice (lmoe_expert_kernel); every choice computes the same layer
EXPERTS_AUTO, EXPERTS_TILED, EXPERTS_STREAM, EXPERTS_FUSED = 0, 1, 2, 3
_EXPERT_KERNEL = {"auto": EXPERTS_AUTO, "tiled": EXPERTS_TILED, "stream": EXPERTS_STREAM,
                  "fused": EXPERTS_FUSED}
NUM_STAGES = 8
STAGE_NAMES = ("down_router", "topk", "dispatch", "fc1", "fc2", "combine", "up", "shared")

_DT = {"f32": LMOE_F32, "bf16": LMOE_BF16, "fp8_e4m3_rowscale": LMOE_FP8_E4M3_ROWSCALE,
       "mxfp4_e2m1": LMOE_MXFP4_E2M1}
_GATE = {"softmax_all": GATE_SOFTMAX_ALL, "softmax_topk": GATE_SOFTMAX_TOPK,
         "sigmoid_topk_norm": GATE_SIGMOID_TOPK_NORM}

EXPORTED = ("latentmoe_create", "latentmoe_workspace_size", "latentmoe_forward",
            "latentmoe_destroy", "latentmoe_timer_create", "latentmoe_timer_read",
            "latentmoe_timer_destroy", "latentmoe_status_string", "latentmoe_last_error",
            "latentmoe_expert_regime", "latentmoe_overlap_create", "latentmoe_overlap_destroy",
            "latentmoe_forward_overlap", "latentmoe_forward_static",
            "latentmoe_packed_weights_size", "latentmoe_pack_expert_weights")


class LmoeConfig(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("l", ctypes.c_int64), ("m", ctypes.c_int64),
                ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("router_input", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("expert_dtype", ctypes.c_int32), ("has_projections", ctypes.c_int32),
                ("has_router_bias", ctypes.c_int32), ("expert_kernel", ctypes.c_int32),
                ("n_shared", ctypes.c_int64), ("m_shared", ctypes.c_int64)]


class LmoeWeights(ctypes.Structure):
    _fields_ = [("w_down", ctypes.c_void_p), ("w_router", ctypes.c_void_p),
                ("router_bias", ctypes.c_void_p), ("w1", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w1_scale", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_shared1", ctypes.c_void_p), ("w_shared2", ctypes.c_void_p),
                ("w1_mx", ctypes.c_void_p), ("w2_mx", ctypes.c_void_p),
                ("experts_packed", ctypes.c_void_p)]


class LmoeDebug(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_gate", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("slot_of", ctypes.c_void_p), ("token_of", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("latent", ctypes.c_void_p),
                ("timer", ctypes.c_void_p)]


class LatentMoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded liblatentmoe.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("liblatentmoe.so is not built (run __graft_entry__.build() or "
                                   "python mixture_experts_layer_32_amd/build.py)")
            # torch carries its own HIP runtime under the same soname as the
            # system one: load it first, so that the library binds to the
            # runtime that owns the tensors' memory (loaded the other way
            # round, the process holds two runtimes and the library's sees
            # no device)
            _torch()
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
            L.latentmoe_create.argtypes = [ctypes.POINTER(LmoeConfig), ctypes.POINTER(vp)]
            L.latentmoe_workspace_size.argtypes = [vp, i64, ctypes.POINTER(ctypes.c_size_t)]
            L.latentmoe_forward.argtypes = [vp, ctypes.POINTER(LmoeWeights), vp, i64, vp,
                                            ctypes.POINTER(LmoeDebug), vp, ctypes.c_size_t, vp]
            L.latentmoe_forward_overlap.argtypes = [vp, ctypes.POINTER(LmoeWeights), vp, i64, vp,
                                                    ctypes.POINTER(LmoeDebug), vp,
                                                    ctypes.c_size_t, vp, vp]
            L.latentmoe_forward_static.argtypes = [vp, ctypes.POINTER(LmoeWeights), vp, i64, vp,
                                                   ctypes.POINTER(LmoeDebug), vp]
            L.latentmoe_overlap_create.argtypes = [vp, ctypes.POINTER(vp)]
            L.latentmoe_overlap_destroy.argtypes = [vp]
            L.latentmoe_destroy.argtypes = [vp]
            L.latentmoe_timer_create.argtypes = [ctypes.POINTER(vp)]
            L.latentmoe_timer_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32,
                                               ctypes.POINTER(i32)]
            L.latentmoe_timer_destroy.argtypes = [vp]
            L.latentmoe_status_string.argtypes = [ctypes.c_int]
            L.latentmoe_status_string.restype = ctypes.c_char_p
            L.latentmoe_last_error.argtypes = []
            L.latentmoe_last_error.restype = ctypes.c_char_p
            L.latentmoe_expert_regime.argtypes = [vp, i64]
            L.latentmoe_expert_regime.restype = ctypes.c_char_p
            L.latentmoe_packed_weights_size.argtypes = [vp]
            L.latentmoe_packed_weights_size.restype = ctypes.c_size_t
            L.latentmoe_pack_expert_weights.argtypes = [vp, ctypes.POINTER(LmoeWeights), vp,
                                                        ctypes.c_size_t, vp]
            for f in ("latentmoe_create", "latentmoe_workspace_size", "latentmoe_forward",
                      "latentmoe_destroy", "latentmoe_timer_create", "latentmoe_timer_read",
                      "latentmoe_timer_destroy", "latentmoe_forward_overlap",
                      "latentmoe_forward_static", "latentmoe_pack_expert_weights",
                      "latentmoe_overlap_create", "latentmoe_overlap_destroy"):
                getattr(L, f).restype = ctypes.c_int
            _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        L = lib()
        raise LatentMoEError(status, "%s: %s" % (L.latentmoe_status_string(status).decode(),
                                                 L.latentmoe_last_error().decode()))


def make_config(spec, expert_kernel: str = "auto") -> LmoeConfig:
    """C config from a LayerSpec-like object (d, l, m, n_experts, top_k, ...).
    expert_kernel: "auto", "tiled", "stream" or "fused" (lmoe_expert_kernel)."""
    return LmoeConfig(spec.d, spec.l, spec.m, spec.n_experts, spec.top_k,
                      ROUTER_ON_LATENT if spec.router_on_latent else ROUTER_ON_X,
                      _GATE[spec.gating], _ACT[getattr(spec, "activation", "sqrelu")],
                      _DT[spec.act_dtype], _DT[spec.expert_dtype],
                      int(spec.has_projections), int(spec.has_router_bias),
                      _EXPERT_KERNEL[expert_kernel], getattr(spec, "n_shared", 0),
                      getattr(spec, "m_shared", 0))


class StageTimer:
    """Per-stage HIP-event timer attached to forward calls (ms per stage)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().latentmoe_timer_create(ctypes.byref(h)))
        self._h = h

    def read(self):
        """(dict stage -> accumulated ms, number of calls); resets the timer."""
        buf = (ctypes.c_float * NUM_STAGES)()
        n = ctypes.c_int32()
        _check(lib().latentmoe_timer_read(self._h, buf, NUM_STAGES, ctypes.byref(n)))
        return {k: float(buf[i]) for i, k in enumerate(STAGE_NAMES)}, int(n.value)

    def close(self):
        if self._h:
            lib().latentmoe_timer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Overlap:
    """A side HIP stream for the shared experts (lmoe_overlap).  The stream
    is a torch.cuda.Stream at the default priority, created here unless one
    is given; one forward call at a time may use the object."""

    def __init__(self, stream=None, device=None):
        torch = _torch()
        self.stream = stream if stream is not None else torch.cuda.Stream(device=device)
        h = ctypes.c_void_p()
        _check(lib().latentmoe_overlap_create(ctypes.c_void_p(self.stream.cuda_stream),
                                              ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().latentmoe_overlap_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _torch():
    import torch
    return torch


class LatentMoELayer:
    """Handle on one layer configuration; weights are passed per call."""

    def __init__(self, spec, expert_kernel: str = "auto"):
        self.spec = spec
        self._cfg = make_config(spec, expert_kernel)
        h = ctypes.c_void_p()
        _check(lib().latentmoe_create(ctypes.byref(self._cfg), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().latentmoe_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, T: int) -> int:
        n = ctypes.c_size_t()
        _check(lib().latentmoe_workspace_size(self._h, T, ctypes.byref(n)))
        return int(n.value)

    def expert_regime(self, T: int) -> str:
        return lib().latentmoe_expert_regime(self._h, T).decode()

    def packed_weights_size(self) -> int:
        """Bytes of the banded copy of W1 and W2 that the grouped bf16 and
        fp8 expert kernels read (0: the layer's experts have none)."""
        return int(lib().latentmoe_packed_weights_size(self._h))

    def pack_expert_weights(self, weights: dict, stream=None):
        """The banded copy of weights["w1"] and weights["w2"] as a device
        uint8 tensor, written on the current (or given) stream.  Put it in
        the weights dict as "experts_packed" for forward calls."""
        torch = _torch()
        n = self.packed_weights_size()
        if n == 0:
            raise LatentMoEError(-2, "this layer's experts have no packed form")
        cw = self.weights_struct(weights)
        dev = weights["w1"].device
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        with torch.cuda.stream(st):   # the buffer belongs to the stream that writes it
            buf = torch.empty((n,), dtype=torch.uint8, device=dev)
        _check(lib().latentmoe_pack_expert_weights(self._h, ctypes.byref(cw),
                                                   ctypes.c_void_p(buf.data_ptr()), n,
                                                   ctypes.c_void_p(st.cuda_stream)))
        return buf

    # ---- argument checks (shapes / dtypes of the device tensors)
    def _expect(self, name, t, shape, dtypes):
        torch = _torch()
        if t is None:
            raise ValueError("%s is required" % name)
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        if t.dtype not in dtypes:
            raise ValueError("%s: dtype %s, expected one of %s" % (name, t.dtype, dtypes))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.device.type != "cuda":
            raise ValueError("%s must be a device tensor" % name)
        return t.data_ptr()

    def weights_struct(self, w: dict) -> LmoeWeights:
        torch = _torch()
        s = self.spec
        act = (torch.float32,) if s.act_dtype == "f32" else (torch.bfloat16,)
        if s.expert_dtype == "f32":
            edt = (torch.float32,)
        elif s.expert_dtype == "bf16":
            edt = (torch.bfloat16,)
        elif s.expert_dtype == "mxfp4_e2m1":
            edt = (torch.uint8,)
        else:
            edt = (torch.uint8, torch.float8_e4m3fn)
        fp4 = s.expert_dtype == "mxfp4_e2m1"   # E2M1 pairs: half the columns, in bytes
        r_in = s.l if s.router_on_latent else s.d
        glu = getattr(s, "activation", "sqrelu") == "swiglu"
        m1 = 2 * s.m if glu else s.m  # W1 rows: (up, gate) pairs with SwiGLU
        if glu and "w_gate" in w:
            raise ValueError("SwiGLU weights go in interleaved: pass pack_gated(weights)")
        cw = LmoeWeights()
        cw.w_router = self._expect("w_router", w.get("w_router"), (s.n_experts, r_in), act)
        cw.w1 = self._expect("w1", w.get("w1"), (s.n_experts, m1, s.l // 2 if fp4 else s.l), edt)
        cw.w2 = self._expect("w2", w.get("w2"), (s.n_experts, s.l, s.m // 2 if fp4 else s.m), edt)
        if fp4:
            cw.w1_mx = self._expect("w1_mx", w.get("w1_mx"), (s.n_experts, m1, s.l // 32),
                                    (torch.uint8,))
            cw.w2_mx = self._expect("w2_mx", w.get("w2_mx"), (s.n_experts, s.l, s.m // 32),
                                    (torch.uint8,))
        if s.has_projections:
            cw.w_down = self._expect("w_down", w.get("w_down"), (s.l, s.d), act)
            cw.w_up = self._expect("w_up", w.get("w_up"), (s.d, s.l), act)
        if s.has_router_bias:
            cw.router_bias = self._expect("router_bias", w.get("router_bias"), (s.n_experts,),
                                          (torch.float32,))
        if s.expert_dtype == "fp8_e4m3_rowscale":
            cw.w1_scale = self._expect("w1_scale", w.get("w1_scale"), (s.n_experts, m1),
                                       (torch.float32,))
            cw.w2_scale = self._expect("w2_scale", w.get("w2_scale"), (s.n_experts, s.l),
                                       (torch.float32,))
        if w.get("experts_packed") is not None:
            cw.experts_packed = self._expect("experts_packed", w["experts_packed"],
                                             (self.packed_weights_size(),), (torch.uint8,))
        S = getattr(s, "n_shared", 0)
        if S:
            hs = S * s.m_shared
            cw.w_shared1 = self._expect("w_shared1", w.get("w_shared1"),
                                        (2 * hs if glu else hs, s.d), act)
            cw.w_shared2 = self._expect("w_shared2", w.get("w_shared2"), (s.d, hs), act)
        return cw

    def forward(self, x, weights, out=None, workspace=None, debug: dict | None = None,
                timer: StageTimer | None = None, stream=None, cweights: LmoeWeights | None = None,
                overlap: Overlap | None = None):
        """out[T][d] = layer(x[T][d]) on the current (or given) HIP stream.

        debug: optional dict of preallocated device tensors keyed like
        lmoe_debug_out (topk_idx, topk_gate, expert_counts, expert_offsets,
        slot_of, token_of, logits, latent).  overlap: run the shared experts
        on that object's side stream (latentmoe_forward_overlap).
        """
        torch = _torch()
        s = self.spec
        act = torch.float32 if s.act_dtype == "f32" else torch.bfloat16
        T = int(x.shape[0])
        xp = self._expect("x", x, (T, s.d), (act,))
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        # tensors made here are allocated on the launch stream, so that the
        # caching allocator does not hand their memory to other work on
        # another stream while the call's kernels still use it
        with torch.cuda.stream(stream):
            if out is None:
                out = torch.empty((T, s.d), dtype=act, device=x.device)
            need = self.workspace_size(T)
            if workspace is None:
                workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
        op = self._expect("out", out, (T, s.d), (act,))
        if workspace.numel() < need:
            raise ValueError("workspace has %d bytes, needs %d" % (workspace.numel(), need))
        cw = cweights if cweights is not None else self.weights_struct(weights)
        dbg = self._debug(debug, timer)
        dbg_p = ctypes.byref(dbg) if dbg is not None else None
        st = ctypes.c_void_p(stream.cuda_stream)
        if overlap is not None:
            _check(lib().latentmoe_forward_overlap(self._h, ctypes.byref(cw), xp, T, op, dbg_p,
                                                   workspace.data_ptr(), workspace.numel(), st,
                                                   overlap._h))
        else:
            _check(lib().latentmoe_forward(self._h, ctypes.byref(cw), xp, T, op, dbg_p,
                                           workspace.data_ptr(), workspace.numel(), st))
        return out

    @staticmethod
    def _debug(debug, timer):
        """lmoe_debug_out of the optional device outputs and timer, or None."""
        if not debug and timer is None:
            return None
        dbg = LmoeDebug()
        for k, v in (debug or {}).items():
            if not hasattr(dbg, k):
                raise ValueError("unknown debug output %r" % k)
            setattr(dbg, k, v.data_ptr())
        if timer is not None:
            dbg.timer = timer._h
        return dbg

    def forward_static(self, x, weights, out, debug: dict | None = None,
                       timer: StageTimer | None = None, stream=None,
                       cweights: LmoeWeights | None = None):
        """latentmoe_forward_static: the layer with the library's own device
        scratch as workspace (no allocation in the call).  `out` is required
        (T x d, act dtype); the shared experts run on the launch stream."""
        torch = _torch()
        s = self.spec
        act = torch.float32 if s.act_dtype == "f32" else torch.bfloat16
        T = int(x.shape[0])
        xp = self._expect("x", x, (T, s.d), (act,))
        op = self._expect("out", out, (T, s.d), (act,))
        cw = cweights if cweights is not None else self.weights_struct(weights)
        dbg = self._debug(debug, timer)
        dbg_p = ctypes.byref(dbg) if dbg is not None else None
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        _check(lib().latentmoe_forward_static(self._h, ctypes.byref(cw), xp, T, op, dbg_p,
                                              ctypes.c_void_p(stream.cuda_stream)))
        return out


def debug_buffers(spec, T: int, device="cuda") -> dict:
    """Device tensors for every debug output of a forward call over T tokens."""
    torch = _torch()
    K, N = spec.top_k, spec.n_experts
    act = torch.float32 if spec.act_dtype == "f32" else torch.bfloat16
    d = {"topk_idx": torch.empty((T, K), dtype=torch.int32, device=device),
         "topk_gate": torch.empty((T, K), dtype=torch.float32, device=device),
         "expert_counts": torch.empty((N,), dtype=torch.int32, device=device),
         "expert_offsets": torch.empty((N + 1,), dtype=torch.int32, device=device),
         "slot_of": torch.empty((T, K), dtype=torch.int32, device=device),
         "token_of": torch.empty((T * K,), dtype=torch.int32, device=device),
         "logits": torch.empty((T, N), dtype=torch.float32, device=device)}
    if spec.has_projections:
        d["latent"] = torch.empty((T, spec.l), dtype=act, device=device)
    return d


def pack_gated(weights: dict) -> dict:
    """SwiGLU weights in the interleaved layout the library reads: W_FC1 and
    W_gate ([N][m][l]) become one [N][2m][l] matrix whose rows alternate
    (up, gate); row scales and the shared experts' matrices likewise.  Works
    on numpy arrays or torch tensors; other keys pass through."""
    if "w_gate" not in weights:
        return dict(weights)
    out = {k: v for k, v in weights.items()
           if k not in ("w_gate", "w_gate_scale", "w_shared_gate", "w_gate_mx")}

    def inter(a, g, axis):
        if hasattr(a, "dim"):                      # torch
            t = _torch().stack([a, g], dim=axis + 1)
            return t.reshape(*a.shape[:axis], 2 * a.shape[axis], *a.shape[axis + 1:])
        import numpy as np
        t = np.stack([a, g], axis=axis + 1)
        return t.reshape(a.shape[:axis] + (2 * a.shape[axis],) + a.shape[axis + 1:])

    out["w1"] = inter(weights["w1"], weights["w_gate"], 1)
    if "w1_scale" in weights:
        out["w1_scale"] = inter(weights["w1_scale"], weights["w_gate_scale"], 1)
    if "w1_mx" in weights:
        out["w1_mx"] = inter(weights["w1_mx"], weights["w_gate_mx"], 1)
    if "w_shared1" in weights:
        out["w_shared1"] = inter(weights["w_shared1"], weights["w_shared_gate"], 0)
    return out


def to_device(arrays: dict, device="cuda") -> dict:
    """numpy inputs from the synthetic generator -> device tensors of the
    storage dtype (bf16 bit patterns become torch.bfloat16; fp8 bytes stay uint8)."""
    torch = _torch()
    import numpy as np
    out = {}
    for k, a in arrays.items():
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        out[k] = t.to(device)
    return out
