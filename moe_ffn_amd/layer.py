"""ctypes binding of libmoe_layer.so (the C ABI in include/moe_layer.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current HIP stream.  If the
library has not been built, loading fails loudly; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

# The in-tree build; MOE_LAYER_LIB may name another build of the same sources.
LIB_PATH = os.environ.get("MOE_LAYER_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe_layer.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_OOM, MOE_ERR_HIP, MOE_ERR_UNSUPPORTED = range(5)
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_OOM", 3: "MOE_ERR_HIP",
                4: "MOE_ERR_UNSUPPORTED"}
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1

# Symbols declared in include/moe_layer.h.
EXPORTS = ("moe_abi_version", "moe_last_error", "moe_layer_create", "moe_layer_create_fp8",
           "moe_layer_create_w8a8", "moe_fp8_quantize_rows", "moe_layer_forward",
           "moe_layer_set_bias", "moe_layer_get_bias", "moe_layer_update_bias",
           "moe_layer_timing_start",
           "moe_layer_timing_stop", "moe_layer_destroy", "moe_stack_create", "moe_stack_forward",
           "moe_stack_capture", "moe_stack_replay", "moe_stack_destroy", "moe_stack_set_eda",
           "moe_stack_forward_routing", "moe_layer_forward_static")
TIMED_SLOTS = ("norm_router", "route_permute", "experts_gate_up", "experts_down", "combine",
               "gather", "quant_act")


class LayerConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("max_tokens", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("rms_gain", ctypes.c_void_p), ("w_router", ctypes.c_void_p),
                ("b_router", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class Fp8Scales(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p)]


class RoutingOut(ctypes.Structure):
    _fields_ = [("sel", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("gather", ctypes.c_void_p),
                ("scatter", ctypes.c_void_p)]


def _out_like(hidden: torch.Tensor, out: torch.Tensor | None) -> torch.Tensor:
    """A new output tensor like `hidden`, or `out` if it has hidden's shape,
    dtype and device and is contiguous (the library writes T * d elements
    through its pointer and cannot check its size)."""
    if out is None:
        return torch.empty_like(hidden)
    if not (out.shape == hidden.shape and out.dtype == hidden.dtype
            and out.device == hidden.device and out.is_contiguous()):
        raise ValueError(f"out: need a contiguous {hidden.dtype} tensor of shape "
                         f"{tuple(hidden.shape)} on {hidden.device}")
    return out


class MoELayerError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the library is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m moe_ffn_amd.build`")
    lib = ctypes.CDLL(p)
    lib.moe_abi_version.restype = ctypes.c_int32
    lib.moe_abi_version.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_layer_create.restype = ctypes.c_int
    lib.moe_layer_create.argtypes = [ctypes.POINTER(LayerConfig), ctypes.POINTER(LayerWeights),
                                     ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    for f in (lib.moe_layer_create_fp8, lib.moe_layer_create_w8a8):
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(LayerConfig), ctypes.POINTER(LayerWeights),
                      ctypes.POINTER(Fp8Scales), ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    lib.moe_fp8_quantize_rows.restype = ctypes.c_int
    lib.moe_fp8_quantize_rows.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_layer_forward.restype = ctypes.c_int
    lib.moe_layer_forward.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.POINTER(RoutingOut)]
    lib.moe_layer_forward_static.restype = ctypes.c_int
    lib.moe_layer_forward_static.argtypes = lib.moe_layer_forward.argtypes
    lib.moe_layer_set_bias.restype = ctypes.c_int
    lib.moe_layer_set_bias.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_layer_get_bias.restype = ctypes.c_int
    lib.moe_layer_get_bias.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_layer_update_bias.restype = ctypes.c_int
    lib.moe_layer_update_bias.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                          ctypes.c_void_p]
    lib.moe_layer_timing_start.restype = ctypes.c_int
    lib.moe_layer_timing_start.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.moe_layer_timing_stop.restype = ctypes.c_int
    lib.moe_layer_timing_stop.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_int32)]
    lib.moe_layer_destroy.restype = None
    lib.moe_layer_destroy.argtypes = [ctypes.c_void_p]
    lib.moe_stack_create.restype = ctypes.c_int
    lib.moe_stack_create.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    for name in ("moe_stack_forward", "moe_stack_capture"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                      ctypes.c_void_p]
    lib.moe_stack_forward_routing.restype = ctypes.c_int
    lib.moe_stack_forward_routing.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.POINTER(RoutingOut)]
    lib.moe_stack_replay.restype = ctypes.c_int
    lib.moe_stack_replay.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_stack_destroy.restype = None
    lib.moe_stack_destroy.argtypes = [ctypes.c_void_p]
    lib.moe_stack_set_eda.restype = ctypes.c_int
    lib.moe_stack_set_eda.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_float]
    if path is None:
        _lib = lib
    return lib


def _check(lib, status: int):
    if status != MOE_OK:
        raise MoELayerError(status, lib.moe_last_error().decode(errors="replace"))


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def fp8_quantize_rows(x: torch.Tensor, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """moe_fp8_quantize_rows: x [R, K] contiguous CUDA bf16 (K % 8 == 0) ->
    (codes [R, K] uint8 E4M3, scales [R] float32), per-row dynamic scales."""
    lib = load_library()
    if not (x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()):
        raise ValueError("x: need a contiguous CUDA bfloat16 tensor [R, K]")
    R, K = x.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((R,), dtype=torch.float32, device=x.device)
    _check(lib, lib.moe_fp8_quantize_rows(ctypes.c_void_p(x.data_ptr()), R, K,
                                          ctypes.c_void_p(codes.data_ptr()),
                                          ctypes.c_void_p(scales.data_ptr()),
                                          ctypes.c_void_p(_stream_ptr(stream))))
    return codes, scales


_TORCH_DTYPE = {MOE_DTYPE_F32: torch.float32, MOE_DTYPE_BF16: torch.bfloat16}


class MoELayer:
    """One MoE FFN layer owned by the library (packed weights + workspace).

    weights: dict of CUDA tensors in canonical row-major layout
      rms_gain [d], w_router [E, d], b_router [E] (fp32), w_gate [E, F, d],
      w_up [E, F, d], w_down [E, d, F]; all but b_router in the layer dtype.
    fp8_scales: None, or a dict of contiguous CUDA float32 per-row scales
      gate [E, F], up [E, F], down [E, d]; then w_gate, w_up and w_down hold
      E4M3 codes (torch.uint8 or torch.float8_e4m3fn) and dtype must be "bf16"
      (moe_layer_create_fp8).
    fp8_act: with fp8_scales, quantise the activations to E4M3 as well
      (moe_layer_create_w8a8: both GEMM operands fp8, per-row dynamic scales).
    """

    def __init__(self, d_model: int, d_ff: int, n_experts: int, top_k: int, dtype: str,
                 weights: dict, max_tokens: int, rms_eps: float = 1e-6, stream=None,
                 fp8_scales: dict | None = None, fp8_act: bool = False):
        self._lib = load_library()
        self.handle = None
        self.dtype_code = MOE_DTYPE_BF16 if dtype == "bf16" else MOE_DTYPE_F32
        self.torch_dtype = _TORCH_DTYPE[self.dtype_code]
        self.d, self.F, self.E, self.k = d_model, d_ff, n_experts, top_k
        self.max_tokens = max_tokens
        shapes = {"rms_gain": (d_model,), "w_router": (n_experts, d_model),
                  "b_router": (n_experts,), "w_gate": (n_experts, d_ff, d_model),
                  "w_up": (n_experts, d_ff, d_model), "w_down": (n_experts, d_model, d_ff)}
        self.fp8 = fp8_scales is not None
        if fp8_act and not self.fp8:
            raise ValueError("fp8_act needs fp8 weights (fp8_scales)")
        self.fp8_act = fp8_act
        ptrs = {}
        for name, shp in shapes.items():
            t = weights[name]
            want = torch.float32 if name == "b_router" else self.torch_dtype
            if self.fp8 and name in ("w_gate", "w_up", "w_down"):
                if t.dtype == torch.float8_e4m3fn:
                    t = t.view(torch.uint8)
                want = torch.uint8
            if not (t.is_cuda and t.dtype == want and tuple(t.shape) == shp and t.is_contiguous()):
                raise ValueError(f"{name}: need a contiguous CUDA {want} tensor of shape {shp}")
            ptrs[name] = t.data_ptr()
        cfg = LayerConfig(d_model, d_ff, n_experts, top_k, self.dtype_code, rms_eps, max_tokens)
        w = LayerWeights(**ptrs)
        h = ctypes.c_void_p()
        stream_p = ctypes.c_void_p(_stream_ptr(stream))
        if self.fp8:
            sshapes = {"gate": (n_experts, d_ff), "up": (n_experts, d_ff),
                       "down": (n_experts, d_model)}
            sptrs = {}
            for name, shp in sshapes.items():
                t = fp8_scales[name]
                if not (t.is_cuda and t.dtype == torch.float32 and tuple(t.shape) == shp
                        and t.is_contiguous()):
                    raise ValueError(f"fp8 scale {name}: need a contiguous CUDA float32 tensor "
                                     f"of shape {shp}")
                sptrs[name] = t.data_ptr()
            sc = Fp8Scales(**sptrs)
            create = (self._lib.moe_layer_create_w8a8 if fp8_act
                      else self._lib.moe_layer_create_fp8)
            _check(self._lib, create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(sc),
                                     stream_p, ctypes.byref(h)))
        else:
            _check(self._lib, self._lib.moe_layer_create(ctypes.byref(cfg), ctypes.byref(w),
                                                         stream_p, ctypes.byref(h)))
        self.handle = h

    def forward(self, hidden: torch.Tensor, out: torch.Tensor | None = None,
                routing: bool = False, stream=None, static_scratch: bool = False):
        """hidden [T, d] -> out [T, d]; with routing=True also returns a dict of
        sel, gate, counts, offsets, gather, scatter (int32 / fp32 CUDA tensors).
        static_scratch=True calls moe_layer_forward_static (the per-call
        buffers in the library's static scratch array instead of the layer's
        workspace; `out` and the routing buffers should then be allocated by
        the caller beforehand when nothing may be allocated)."""
        if self.handle is None:
            raise RuntimeError("layer is closed")
        if not (hidden.is_cuda and hidden.dtype == self.torch_dtype and hidden.dim() == 2
                and hidden.shape[1] == self.d and hidden.is_contiguous()):
            raise ValueError(f"hidden: need a contiguous CUDA {self.torch_dtype} tensor [T, {self.d}]")
        T = hidden.shape[0]
        out = _out_like(hidden, out)
        r = None
        rp = None
        if routing:
            r, rp = self.routing_buffers(T, hidden.device)
        fwd = self._lib.moe_layer_forward_static if static_scratch else self._lib.moe_layer_forward
        st = fwd(self.handle, ctypes.c_void_p(hidden.data_ptr()), T,
                 ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(_stream_ptr(stream)),
                 ctypes.byref(rp) if rp is not None else None)
        _check(self._lib, st)
        return (out, r) if routing else out

    __call__ = forward

    def routing_buffers(self, T: int, dev) -> tuple[dict, RoutingOut]:
        """Fresh routing outputs for a forward over T tokens, and their struct."""
        n = T * self.k
        r = {"sel": torch.empty((T, self.k), dtype=torch.int32, device=dev),
             "gate": torch.empty((T, self.k), dtype=torch.float32, device=dev),
             "counts": torch.empty(self.E, dtype=torch.int32, device=dev),
             "offsets": torch.empty(self.E + 1, dtype=torch.int32, device=dev),
             "gather": torch.empty(n, dtype=torch.int32, device=dev),
             "scatter": torch.empty(n, dtype=torch.int32, device=dev)}
        return r, RoutingOut(**{k: v.data_ptr() for k, v in r.items()})

    def set_bias(self, b: torch.Tensor, stream=None):
        if not (b.is_cuda and b.dtype == torch.float32 and b.numel() == self.E and b.is_contiguous()):
            raise ValueError("bias: need a contiguous CUDA fp32 tensor of n_experts values")
        _check(self._lib, self._lib.moe_layer_set_bias(self.handle, ctypes.c_void_p(b.data_ptr()),
                                                       ctypes.c_void_p(_stream_ptr(stream))))

    def get_bias(self, stream=None) -> torch.Tensor:
        """The layer's current router bias (fp32 CUDA tensor of n_experts values)."""
        b = torch.empty(self.E, dtype=torch.float32, device="cuda")
        _check(self._lib, self._lib.moe_layer_get_bias(self.handle, ctypes.c_void_p(b.data_ptr()),
                                                       ctypes.c_void_p(_stream_ptr(stream))))
        return b

    def update_bias(self, rate: float, counts: torch.Tensor | None = None, stream=None):
        """One balancing step b_e += rate * sign(mean(c) - c_e) on the layer's bias.

        counts: int32 CUDA tensor of n_experts counts (e.g. routing["counts"] of
        a forward), or None for the counts of the latest forward that did not
        return its routing counts."""
        ptr = None
        if counts is not None:
            if not (counts.is_cuda and counts.dtype == torch.int32 and counts.numel() == self.E
                    and counts.is_contiguous()):
                raise ValueError("counts: need a contiguous CUDA int32 tensor of n_experts values")
            ptr = ctypes.c_void_p(counts.data_ptr())
        _check(self._lib, self._lib.moe_layer_update_bias(self.handle, ptr, ctypes.c_float(rate),
                                                          ctypes.c_void_p(_stream_ptr(stream))))

    def timing_start(self, max_forwards: int):
        """Record per-kernel HIP events in the next `max_forwards` forwards."""
        _check(self._lib, self._lib.moe_layer_timing_start(self.handle, int(max_forwards)))

    def timing_stop(self) -> tuple[dict, int]:
        """Wait for the recorded events; return ({slot: summed ms}, forwards recorded)."""
        ms = (ctypes.c_float * len(TIMED_SLOTS))()
        n = ctypes.c_int32()
        _check(self._lib, self._lib.moe_layer_timing_stop(self.handle, ms, ctypes.byref(n)))
        return {name: float(ms[i]) for i, name in enumerate(TIMED_SLOTS)}, int(n.value)

    def close(self):
        if self.handle is not None:
            self._lib.moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MoEStack:
    """The FFN half of a stack of layers with residual adds, run by the library:
    h_{l+1} = h_l + layer_l(h_l).  The MoELayer objects are borrowed and must
    stay alive (and open) while the stack is used."""

    def __init__(self, layers: list, max_tokens: int):
        self._lib = load_library()
        self.handle = None
        if not layers:
            raise ValueError("a stack needs at least one layer")
        self.layers = list(layers)
        self.d, self.torch_dtype, self.max_tokens = layers[0].d, layers[0].torch_dtype, max_tokens
        arr = (ctypes.c_void_p * len(layers))(*[L.handle.value for L in layers])
        h = ctypes.c_void_p()
        _check(self._lib, self._lib.moe_stack_create(len(layers), arr, int(max_tokens),
                                                     ctypes.byref(h)))
        self.handle = h

    def _io(self, hidden: torch.Tensor, out):
        if not (hidden.is_cuda and hidden.dtype == self.torch_dtype and hidden.dim() == 2
                and hidden.shape[1] == self.d and hidden.is_contiguous()):
            raise ValueError(f"hidden: need a contiguous CUDA {self.torch_dtype} tensor [T, {self.d}]")
        return _out_like(hidden, out)

    def forward(self, hidden: torch.Tensor, out: torch.Tensor | None = None, stream=None):
        out = self._io(hidden, out)
        _check(self._lib, self._lib.moe_stack_forward(self.handle, ctypes.c_void_p(hidden.data_ptr()),
                                                      hidden.shape[0], ctypes.c_void_p(out.data_ptr()),
                                                      ctypes.c_void_p(_stream_ptr(stream))))
        return out

    __call__ = forward

    def forward_routing(self, hidden: torch.Tensor, out: torch.Tensor | None = None, stream=None):
        """One pass that also returns every layer's routing (a list of dicts as
        from MoELayer.forward(routing=True)); see moe_stack_forward_routing."""
        out = self._io(hidden, out)
        T = hidden.shape[0]
        bufs = [L.routing_buffers(T, hidden.device) for L in self.layers]
        arr = (RoutingOut * len(bufs))(*[b[1] for b in bufs])
        _check(self._lib, self._lib.moe_stack_forward_routing(
            self.handle, ctypes.c_void_p(hidden.data_ptr()), T, ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(_stream_ptr(stream)), arr))
        return out, [b[0] for b in bufs]

    def capture(self, hidden: torch.Tensor, out: torch.Tensor, stream):
        """Record one pass (these pointers, this T) into the stack's HIP graph."""
        out = self._io(hidden, out)
        _check(self._lib, self._lib.moe_stack_capture(self.handle, ctypes.c_void_p(hidden.data_ptr()),
                                                      hidden.shape[0], ctypes.c_void_p(out.data_ptr()),
                                                      ctypes.c_void_p(_stream_ptr(stream))))

    def replay(self, stream=None):
        _check(self._lib, self._lib.moe_stack_replay(self.handle, ctypes.c_void_p(_stream_ptr(stream))))

    def set_eda(self, alpha: float | None):
        """Depth-average the router logits across the MoE layers at rate alpha
        (None: off); see moe_stack_set_eda."""
        _check(self._lib, self._lib.moe_stack_set_eda(self.handle, 0 if alpha is None else 1,
                                                      0.0 if alpha is None else float(alpha)))

    def close(self):
        if self.handle is not None:
            self._lib.moe_stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
