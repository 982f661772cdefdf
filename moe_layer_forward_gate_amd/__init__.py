"""Python binding of libmoe (the MoE layer forward on MI355X).

Argument marshalling only: every step of the forward runs in libmoe's HIP
kernels. The raw C entry points keep their C names (moe_layer_create,
moe_forward, moe_forward_routed, moe_set_profiling, moe_stage_times, moe_destroy, moe_status_str,
moe_last_error);
MoeLayer wraps them for torch device tensors. PyTorch supplies device memory and
streams. If libmoe.so has not been built, loading raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

__all__ = [
    "MoeError", "lib", "MOE_F32", "MOE_BF16", "MOE_I8", "MOE_I4", "MOE_WEIGHT_SOFTMAX", "MOE_WEIGHT_RAW", "MoeDesc", "MoeWeights", "MoeRouteOut",
    "moe_layer_create", "moe_forward", "moe_forward_routed", "moe_forward_noalloc", "MOE_STATIC_SCRATCH_BYTES", "moe_set_profiling", "moe_stage_times",
    "moe_destroy", "moe_status_str", "moe_last_error", "MoeLayer", "check_weight_tensors", "LIB_PATH", "EXPORTED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOMEM, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_I8, MOE_I4 = 0, 1, 2, 3
MOE_WEIGHT_SOFTMAX, MOE_WEIGHT_RAW = 0, 1

# every symbol include/moe.h declares
EXPORTED = ("moe_layer_create", "moe_forward", "moe_forward_routed", "moe_forward_noalloc", "moe_set_profiling",
            "moe_stage_times", "moe_destroy", "moe_status_str", "moe_last_error")
MOE_STATIC_SCRATCH_BYTES = 64 << 20  # the static scratch of moe_forward_noalloc, per device


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status} ({moe_status_str(status)}): {message}")
        self.status = status


class MoeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_model", "n_experts", "d_ff", "top_k", "max_tokens", "act_dtype", "expert_dtype",
        "shared_d_ff", "profile", "gate_clamp", "gate_weighting")]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "b_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "w_shared_gate", "ws_gate", "ws_up", "ws_down")]


class MoeRouteOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_idx", "topk_w", "expert_counts", "expert_offsets", "sorted_assign", "shared_gate")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmoe.so not found at {LIB_PATH}; build it with "
                              "`python -m moe_layer_forward_gate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_layer_create.argtypes = [ctypes.POINTER(MoeDesc), ctypes.POINTER(MoeWeights),
                                       ctypes.POINTER(ctypes.c_void_p)]
        L.moe_layer_create.restype = ctypes.c_int
        L.moe_forward.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.POINTER(MoeRouteOut), ctypes.c_void_p]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward_routed.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.POINTER(MoeRouteOut), ctypes.c_void_p]
        L.moe_forward_routed.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = L.moe_forward.argtypes
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_set_profiling.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.moe_set_profiling.restype = ctypes.c_int
        L.moe_stage_times.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
        L.moe_stage_times.restype = ctypes.c_int
        L.moe_destroy.argtypes = [ctypes.c_void_p]
        L.moe_destroy.restype = None
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where, moe_last_error())


def moe_layer_create(desc: MoeDesc, weights: MoeWeights) -> ctypes.c_void_p:
    """Raw create; returns the opaque handle or raises MoeError."""
    h = ctypes.c_void_p()
    _check(lib().moe_layer_create(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(h)),
           "moe_layer_create")
    return h


def moe_forward(handle, x_ptr: int, T: int, y_ptr: int, route: MoeRouteOut, stream_ptr: int = 0) -> None:
    """Raw forward on device pointers; enqueues on the given HIP stream."""
    _check(lib().moe_forward(handle, x_ptr, T, y_ptr, ctypes.byref(route), stream_ptr), "moe_forward")


def moe_forward_noalloc(handle, x_ptr: int, T: int, y_ptr: int, route: MoeRouteOut, stream_ptr: int = 0) -> None:
    """Raw forward in the library's static scratch (allocates nothing); as moe_forward."""
    _check(lib().moe_forward_noalloc(handle, x_ptr, T, y_ptr, ctypes.byref(route), stream_ptr),
           "moe_forward_noalloc")


def moe_forward_routed(handle, x_ptr: int, T: int, idx_ptr: int, w_ptr: int, shared_gate_ptr: int, y_ptr: int,
                       route: Optional[MoeRouteOut] = None, stream_ptr: int = 0) -> None:
    """Raw forward with a given routing (topk_idx [T][k] int32, topk_w [T][k] fp32,
    shared_gate [T] fp32 or 0); route may be None."""
    _check(lib().moe_forward_routed(handle, x_ptr, T, idx_ptr, w_ptr, shared_gate_ptr or None, y_ptr,
                                    ctypes.byref(route) if route is not None else None, stream_ptr),
           "moe_forward_routed")


def moe_set_profiling(handle, enable: bool) -> None:
    _check(lib().moe_set_profiling(handle, 1 if enable else 0), "moe_set_profiling")


def moe_stage_times(handle):
    ms = (ctypes.c_float * 5)()
    _check(lib().moe_stage_times(handle, ms), "moe_stage_times")
    return list(ms)


def moe_destroy(handle) -> None:
    lib().moe_destroy(handle)


# ---------------------------------------------------------------- torch wrapper
@dataclass
class RouteResult:
    y: "object"
    topk_idx: "object"
    topk_w: "object"
    expert_counts: Optional["object"] = None
    expert_offsets: Optional["object"] = None
    sorted_assign: Optional["object"] = None
    shared_gate: Optional["object"] = None


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def check_weight_tensors(tensors: dict, expected: dict, device) -> None:
    """Raise ValueError unless every tensor matches `expected` (MoeLayer.expected_weights):
    present exactly when expected, contiguous, on `device`, of an accepted dtype and the
    exact shape."""
    for name, want in expected.items():
        t = tensors.get(name)
        if want is None:
            if t is not None:
                raise ValueError(f"{name} given but this layer shape does not take it")
            continue
        if t is None:
            raise ValueError(f"{name} is required for this layer shape")
        dts, shape = want
        if t.device != device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on {device}")
        if t.dtype not in dts or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {' or '.join(str(x) for x in dts)} of shape {shape}, "
                             f"got {t.dtype} {tuple(t.shape)}")


class MoeLayer:
    """One MoE layer held by libmoe on the current GPU.

    Weights are torch tensors on that GPU in the layouts include/moe.h states
    (w_gate/w_up [E, d, F], w_down [E, F, d], w_router [d, E], ...); they are
    copied into libmoe's packed layout, so they may be freed afterwards.
    """

    _DT = {"f32": MOE_F32, "bf16": MOE_BF16, "i8": MOE_I8, "i4": MOE_I4}
    _WEIGHTING = {"softmax": MOE_WEIGHT_SOFTMAX, "raw": MOE_WEIGHT_RAW}

    @staticmethod
    def expected_weights(d_model, n_experts, d_ff, act_dtype, expert_dtype, shared_d_ff=0, has_bias=False):
        """{name: (torch dtypes accepted, shape)} of every weight tensor the layer reads
        (the layouts include/moe.h states); None marks a tensor that must be absent."""
        import torch
        d, E, F = d_model, n_experts, d_ff
        wdt = {"f32": (torch.float32,), "bf16": (torch.bfloat16,), "i8": (torch.int8,),
               "i4": (torch.uint8, torch.int8)}[expert_dtype]
        f32 = (torch.float32,)
        if expert_dtype == "i4":  # two values a byte along the input axis, group scales
            exp = dict(w_gate=(wdt, (E, d // 2, F)), w_up=(wdt, (E, d // 2, F)), w_down=(wdt, (E, F // 2, d)),
                       s_gate=(f32, (E, d // 128, F)), s_up=(f32, (E, d // 128, F)),
                       s_down=(f32, (E, F // 128, d)))
        else:
            exp = dict(w_gate=(wdt, (E, d, F)), w_up=(wdt, (E, d, F)), w_down=(wdt, (E, F, d)))
            if expert_dtype == "i8":
                exp.update(s_gate=(f32, (E, F)), s_up=(f32, (E, F)), s_down=(f32, (E, d)))
            else:
                exp.update(s_gate=None, s_up=None, s_down=None)
        exp["w_router"] = (f32, (d, E))
        exp["b_router"] = (f32, (E,)) if has_bias else None
        if shared_d_ff:
            bf = (torch.bfloat16,)
            exp.update(w_shared_gate=(f32, (d,)), ws_gate=(bf, (d, shared_d_ff)), ws_up=(bf, (d, shared_d_ff)),
                       ws_down=(bf, (shared_d_ff, d)))
        else:
            exp.update(w_shared_gate=None, ws_gate=None, ws_up=None, ws_down=None)
        return exp

    def __init__(self, *, d_model: int, n_experts: int, d_ff: int, top_k: int, max_tokens: int,
                 act_dtype: str, expert_dtype: str, w_router, w_gate, w_up, w_down, b_router=None,
                 s_gate=None, s_up=None, s_down=None, shared_d_ff: int = 0, w_shared_gate=None,
                 ws_gate=None, ws_up=None, ws_down=None, profile: bool = False, gate_clamp: bool = False,
                 gate_weighting: str = "softmax"):
        import torch
        self.torch = torch
        self.d_model, self.n_experts, self.d_ff, self.top_k = d_model, n_experts, d_ff, top_k
        self.max_tokens, self.shared_d_ff = max_tokens, shared_d_ff
        self.act_dtype = act_dtype
        self._act_torch = torch.float32 if act_dtype == "f32" else torch.bfloat16
        tensors = dict(w_router=w_router, b_router=b_router, w_gate=w_gate, w_up=w_up, w_down=w_down,
                       s_gate=s_gate, s_up=s_up, s_down=s_down, w_shared_gate=w_shared_gate,
                       ws_gate=ws_gate, ws_up=ws_up, ws_down=ws_down)
        if act_dtype not in ("f32", "bf16") or expert_dtype not in self._DT:
            raise ValueError(f"unknown dtypes act={act_dtype!r} expert={expert_dtype!r}")
        if gate_weighting not in self._WEIGHTING:
            raise ValueError(f"gate_weighting must be one of {sorted(self._WEIGHTING)}")
        # every tensor's dtype, shape and device is checked here, before the library reads
        # the bytes that the layout implies from its pointer
        exp = self.expected_weights(d_model, n_experts, d_ff, act_dtype, expert_dtype, shared_d_ff,
                                    has_bias=b_router is not None)
        check_weight_tensors(tensors, exp, torch.device("cuda", torch.cuda.current_device()))
        desc = MoeDesc(d_model, n_experts, d_ff, top_k, max_tokens, self._DT[act_dtype],
                       self._DT[expert_dtype], shared_d_ff, 1 if profile else 0, 1 if gate_clamp else 0,
                       self._WEIGHTING[gate_weighting])
        w = MoeWeights(*[_ptr(tensors[f]) for f, _ in MoeWeights._fields_])
        self._h = moe_layer_create(desc, w)

    def close(self) -> None:
        if getattr(self, "_h", None):
            moe_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def outputs(self, T: int, scatter: bool = False):
        """Freshly allocated output buffers for T tokens (allocation is the caller's)."""
        torch = self.torch
        dev = torch.device("cuda", torch.cuda.current_device())
        r = RouteResult(
            y=torch.empty((T, self.d_model), dtype=self._act_torch, device=dev),
            topk_idx=torch.empty((T, self.top_k), dtype=torch.int32, device=dev),
            topk_w=torch.empty((T, self.top_k), dtype=torch.float32, device=dev))
        if scatter:
            r.expert_counts = torch.empty(self.n_experts, dtype=torch.int32, device=dev)
            r.expert_offsets = torch.empty(self.n_experts + 1, dtype=torch.int32, device=dev)
            r.sorted_assign = torch.empty(T * self.top_k, dtype=torch.int32, device=dev)
            if self.shared_d_ff:
                r.shared_gate = torch.empty(T, dtype=torch.float32, device=dev)
        return r

    def forward(self, x, out: Optional[RouteResult] = None, scatter: bool = False, stream=None,
                noalloc: bool = False) -> RouteResult:
        """Enqueue the layer on `stream` (default: torch's current stream) and return the outputs.
        noalloc: run moe_forward_noalloc (the library's static scratch instead of the layer's
        workspace; pass `out` to allocate nothing here either)."""
        torch = self.torch
        if x.dim() != 2 or x.shape[1] != self.d_model or x.dtype != self._act_torch:
            raise ValueError(f"x must be [T, {self.d_model}] {self._act_torch}")
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError("x must be a contiguous GPU tensor")
        T = x.shape[0]
        if out is None:
            out = self.outputs(T, scatter)
        route = MoeRouteOut(_ptr(out.topk_idx), _ptr(out.topk_w), _ptr(out.expert_counts),
                            _ptr(out.expert_offsets), _ptr(out.sorted_assign), _ptr(out.shared_gate))
        s = stream if stream is not None else torch.cuda.current_stream()
        (moe_forward_noalloc if noalloc else moe_forward)(self._h, _ptr(x), T, _ptr(out.y), route,
                                                           int(s.cuda_stream))
        return out

    def forward_routed(self, x, topk_idx, topk_w, shared_gate=None, out: Optional[RouteResult] = None,
                       scatter: bool = False, stream=None) -> RouteResult:
        """Enqueue the layer with the routing given (topk_idx [T, k] int32, topk_w [T, k]
        float32, shared_gate [T] float32 for a layer with a shared expert) instead of the
        gate. The returned RouteResult holds y (and the scatter tables if `scatter`); its
        topk_idx / topk_w are the given tensors."""
        torch = self.torch
        if x.dim() != 2 or x.shape[1] != self.d_model or x.dtype != self._act_torch:
            raise ValueError(f"x must be [T, {self.d_model}] {self._act_torch}")
        T = x.shape[0]
        for name, t, dt, shape in (("topk_idx", topk_idx, torch.int32, (T, self.top_k)),
                                   ("topk_w", topk_w, torch.float32, (T, self.top_k)),
                                   ("shared_gate", shared_gate, torch.float32, (T,))):
            if t is None:
                continue
            if tuple(t.shape) != shape or t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous GPU {dt} tensor of shape {shape}")
        for name, t in (("x", x),):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous GPU tensor")
        if out is None:
            out = self.outputs(T, scatter)
            out.topk_idx, out.topk_w, out.shared_gate = topk_idx, topk_w, shared_gate
        route = MoeRouteOut(0, 0, _ptr(out.expert_counts), _ptr(out.expert_offsets), _ptr(out.sorted_assign), 0)
        s = stream if stream is not None else torch.cuda.current_stream()
        moe_forward_routed(self._h, _ptr(x), T, _ptr(topk_idx), _ptr(topk_w), _ptr(shared_gate), _ptr(out.y),
                           route, int(s.cuda_stream))
        return out

    def set_profiling(self, enable: bool) -> None:
        """Record per-stage HIP events in the following forwards (or stop)."""
        moe_set_profiling(self._h, enable)

    def stage_times(self):
        """[gate, scatter, up, down, combine] ms of the last forward run with profiling on."""
        return moe_stage_times(self._h)
