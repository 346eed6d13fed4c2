"""Python binding of libssm_adjoint.so (the MI355X selective-SSM adjoint-gradient library).

Argument marshalling only: torch provides device memory and the current
stream; every step of the computation runs in the library's HIP kernels.  The
entry points keep the C names (ssm_forward, ssm_adjoint_grad, ssm_stack_grad,
ssm_workspace_bytes, ...).  Importing this module raises if the library has
not been built -- there is no fallback path.

Before a tensor's address crosses the ABI, the binding checks that it lives
on a GPU, is contiguous, has the dtype the call expects (the io dtype for x
and the weights, float32 or float64 elsewhere) and the element count the
dims imply; a mismatch raises SsmError(SSM_ERR_ARG) and nothing is launched
(the library itself sees only pointers and cannot tell a short buffer).

Method: gradient of a diagonal selective state-space layer as the sum of
per-token vector-Jacobian products driven by adjoint states, optionally
truncated to a window (review of "Adjoint sharding for very long context
training of state space models", Core claim: Propositions 2 and 3 and
truncated adjoint sharding).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_adjoint.so")

SSM_F32, SSM_BF16 = 0, 1
STATUS = {0: "SSM_OK", 1: "SSM_ERR_ARG", 2: "SSM_ERR_WORKSPACE", 3: "SSM_ERR_HIP", 4: "SSM_ERR_UNSUPPORTED"}

EXPORTED = (
    "ssm_version",
    "ssm_status_str",
    "ssm_saved_bytes",
    "ssm_sub_state_bytes",
    "ssm_all_state_bytes",
    "ssm_grad_workspace_bytes_sub",
    "ssm_grad_slab_count",
    "ssm_workspace_bytes",
    "ssm_stack_workspace_bytes",
    "ssm_forward",
    "ssm_adjoint_grad",
    "ssm_adjoint_grad_noalloc",
    "ssm_stack_grad",
    "ssm_forward_timed",
    "ssm_adjoint_grad_timed",
    # ssm_probe.h: issue-rate probes of single gfx950 units (no part of the gradient path)
    "ssm_probe_units",
    "ssm_probe_wall_clock_khz",
)

SSM_PROBE_FMA, SSM_PROBE_EXP, SSM_PROBE_EXP_FMA, SSM_PROBE_MFMA = 0, 1, 2, 3
SSM_PROBE_WAVES_PER_WG = 4


class SsmError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, code)}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("P", ctypes.c_int64), ("N", ctypes.c_int64),
                ("chunk", ctypes.c_int32), ("io", ctypes.c_int32)]


class Layer(ctypes.Structure):
    _fields_ = [("W_delta", ctypes.c_void_p), ("W_B", ctypes.c_void_p), ("W_C", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p), ("delta_bias", ctypes.c_void_p), ("norm_scale", ctypes.c_void_p)]


class Saved(ctypes.Structure):
    _fields_ = [("s", ctypes.c_void_p), ("b", ctypes.c_void_p), ("c", ctypes.c_void_p),
                ("h_ckpt", ctypes.c_void_p), ("s_sum", ctypes.c_void_p), ("h_sub", ctypes.c_void_p),
                ("h_all", ctypes.c_void_p)]


class Grads(ctypes.Structure):
    _fields_ = [("dW_delta", ctypes.c_void_p), ("dW_B", ctypes.c_void_p), ("dW_C", ctypes.c_void_p),
                ("dalpha", ctypes.c_void_p), ("dbias", ctypes.c_void_p), ("dx", ctypes.c_void_p),
                ("dnorm_scale", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(python adjoint_gradients_amd/_build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.ssm_version.argtypes = []
    lib.ssm_version.restype = ctypes.c_int32
    lib.ssm_status_str.argtypes = [ctypes.c_int]
    lib.ssm_status_str.restype = ctypes.c_char_p
    lib.ssm_saved_bytes.argtypes = [P(Dims)]
    lib.ssm_saved_bytes.restype = ctypes.c_size_t
    lib.ssm_sub_state_bytes.argtypes = [P(Dims)]
    lib.ssm_sub_state_bytes.restype = ctypes.c_size_t
    lib.ssm_all_state_bytes.argtypes = [P(Dims)]
    lib.ssm_all_state_bytes.restype = ctypes.c_size_t
    lib.ssm_grad_workspace_bytes_sub.argtypes = [P(Dims), ctypes.c_int64]
    lib.ssm_grad_workspace_bytes_sub.restype = ctypes.c_size_t
    lib.ssm_workspace_bytes.argtypes = [P(Dims), ctypes.c_int64, ctypes.c_int32]
    lib.ssm_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_stack_workspace_bytes.argtypes = [ctypes.c_int32, P(Dims), P(Layer), ctypes.c_int64]
    lib.ssm_stack_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_grad_slab_count.argtypes = [P(Dims), ctypes.c_int64, ctypes.c_int32]
    lib.ssm_grad_slab_count.restype = ctypes.c_int32
    lib.ssm_forward.argtypes = [P(Dims), P(Layer), ctypes.c_void_p, ctypes.c_void_p, P(Saved),
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.ssm_forward.restype = ctypes.c_int
    lib.ssm_adjoint_grad.argtypes = [P(Dims), P(Layer), ctypes.c_void_p, P(Saved), ctypes.c_void_p,
                                     ctypes.c_int64, P(Grads), ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
    lib.ssm_adjoint_grad.restype = ctypes.c_int
    lib.ssm_adjoint_grad_noalloc.argtypes = [P(Dims), P(Layer), ctypes.c_void_p, P(Saved), ctypes.c_void_p,
                                             ctypes.c_int64, P(Grads), ctypes.c_void_p]
    lib.ssm_adjoint_grad_noalloc.restype = ctypes.c_int
    lib.ssm_stack_grad.argtypes = [ctypes.c_int32, P(Dims), P(Layer), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, P(Grads), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.ssm_stack_grad.restype = ctypes.c_int
    VP = ctypes.POINTER(ctypes.c_void_p)
    lib.ssm_forward_timed.argtypes = lib.ssm_forward.argtypes + [VP, ctypes.c_int32]
    lib.ssm_forward_timed.restype = ctypes.c_int
    lib.ssm_adjoint_grad_timed.argtypes = lib.ssm_adjoint_grad.argtypes + [VP, ctypes.c_int32]
    lib.ssm_adjoint_grad_timed.restype = ctypes.c_int
    lib.ssm_probe_units.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.ssm_probe_units.restype = ctypes.c_int
    lib.ssm_probe_wall_clock_khz.argtypes = [P(ctypes.c_int)]
    lib.ssm_probe_wall_clock_khz.restype = ctypes.c_int
    return lib


lib = _load()


# ---------------------------------------------------------------- thin wrappers (C names)

def ssm_version() -> int:
    return int(lib.ssm_version())


def ssm_status_str(code: int) -> str:
    return lib.ssm_status_str(code).decode()


def ssm_saved_bytes(dims: Dims) -> int:
    return int(lib.ssm_saved_bytes(ctypes.byref(dims)))


def ssm_sub_state_bytes(dims: Dims) -> int:
    return int(lib.ssm_sub_state_bytes(ctypes.byref(dims)))


def ssm_all_state_bytes(dims: Dims) -> int:
    return int(lib.ssm_all_state_bytes(ctypes.byref(dims)))


def ssm_grad_workspace_bytes_sub(dims: Dims, window: int) -> int:
    return int(lib.ssm_grad_workspace_bytes_sub(ctypes.byref(dims), int(window)))


def ssm_workspace_bytes(dims: Dims, window: int = 0, K: int = 0) -> int:
    return int(lib.ssm_workspace_bytes(ctypes.byref(dims), int(window), int(K)))


def ssm_stack_workspace_bytes(K: int, dims: Dims, layers, window: int) -> int:
    arr = (Layer * K)(*layers)
    return int(lib.ssm_stack_workspace_bytes(int(K), ctypes.byref(dims), arr, int(window)))


def ssm_grad_slab_count(dims: Dims, window: int, sub_states_given: bool) -> int:
    return int(lib.ssm_grad_slab_count(ctypes.byref(dims), int(window), 1 if sub_states_given else 0))


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _need(t, name: str, numel: int, dtype, optional: bool = False, at_least: bool = False):
    """Checks a tensor before its address is passed to the library."""
    import torch

    if t is None:
        if optional:
            return
        raise SsmError(1, f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise SsmError(1, f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise SsmError(1, f"{name}: must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise SsmError(1, f"{name}: must be contiguous")
    if t.dtype != dtype:
        raise SsmError(1, f"{name}: dtype {t.dtype}, expected {dtype}")
    n = t.numel()
    if (n < numel) if at_least else (n != numel):
        raise SsmError(1, f"{name}: {n} elements, expected {'at least ' if at_least else ''}{numel}")


def _io(dims: Dims):
    import torch

    return torch.bfloat16 if dims.io == SSM_BF16 else torch.float32


def _nchunks(dims: Dims) -> int:
    return (dims.T + dims.chunk - 1) // dims.chunk


def _check_ws(ws, ws_bytes: int):
    import torch

    _need(ws, "workspace", int(ws_bytes), torch.uint8, at_least=True)


def _stream(stream) -> int | None:
    if stream is not None:
        return int(stream)
    import torch

    return int(torch.cuda.current_stream().cuda_stream)


def _check(code: int, where: str):
    if code != 0:
        raise SsmError(code, where)


def make_dims(T: int, P: int, N: int, chunk: int = 256, io: str = "f32") -> Dims:
    return Dims(T, P, N, chunk, SSM_BF16 if io == "bf16" else SSM_F32)


def layer_struct(dims: Dims, W_delta, W_B, W_C, alpha, delta_bias=None, norm_scale=None) -> Layer:
    import torch

    P, N, io = dims.P, dims.N, _io(dims)
    _need(W_delta, "W_delta", P * P, io)
    _need(W_B, "W_B", N * P, io)
    _need(W_C, "W_C", N * P, io)
    _need(alpha, "alpha", P * N, torch.float32)
    _need(delta_bias, "delta_bias", P, torch.float32, optional=True)
    _need(norm_scale, "norm_scale", P, torch.float32, optional=True)
    return Layer(_ptr(W_delta), _ptr(W_B), _ptr(W_C), _ptr(alpha), _ptr(delta_bias), _ptr(norm_scale))


def saved_struct(saved: dict, dims: Dims) -> Saved:
    import torch

    T, P, N, K = dims.T, dims.P, dims.N, _nchunks(dims)
    f32 = torch.float32
    _need(saved.get("s"), "saved s", T * P, f32)
    _need(saved.get("b"), "saved b", T * N, f32)
    _need(saved.get("c"), "saved c", T * N, f32)
    _need(saved.get("h_ckpt"), "saved h_ckpt", K * P * N, f32)
    _need(saved.get("s_sum"), "saved s_sum", K * P, torch.float64)
    if saved.get("h_sub") is not None:
        _need(saved["h_sub"], "saved h_sub", ssm_sub_state_bytes(dims) // 4, f32, at_least=True)
    if saved.get("h_all") is not None:
        _need(saved["h_all"], "saved h_all", ssm_all_state_bytes(dims) // 4, f32, at_least=True)
    return Saved(_ptr(saved["s"]), _ptr(saved["b"]), _ptr(saved["c"]), _ptr(saved["h_ckpt"]),
                 _ptr(saved["s_sum"]), _ptr(saved.get("h_sub")), _ptr(saved.get("h_all")))


def grads_struct(grads: dict, dims: Dims) -> Grads:
    import torch

    T, P, N = dims.T, dims.P, dims.N
    f32 = torch.float32
    _need(grads.get("dW_delta"), "dW_delta", P * P, f32)
    _need(grads.get("dW_B"), "dW_B", N * P, f32)
    _need(grads.get("dW_C"), "dW_C", N * P, f32)
    _need(grads.get("dalpha"), "dalpha", P * N, f32, optional=True)
    _need(grads.get("dbias"), "dbias", P, f32, optional=True)
    _need(grads.get("dx"), "dx", T * P, f32, optional=True)
    _need(grads.get("dnorm_scale"), "dnorm_scale", P, f32, optional=True)
    return Grads(_ptr(grads.get("dW_delta")), _ptr(grads.get("dW_B")), _ptr(grads.get("dW_C")),
                 _ptr(grads.get("dalpha")), _ptr(grads.get("dbias")), _ptr(grads.get("dx")),
                 _ptr(grads.get("dnorm_scale")))


def ssm_forward(dims: Dims, layer: Layer, x, y, saved: Saved, ws, ws_bytes: int, stream=None):
    """layer and saved come from LayerTensors.struct / saved_struct, which check their tensors."""
    import torch

    _need(x, "x", dims.T * dims.P, _io(dims))
    _need(y, "y", dims.T * dims.P, torch.float32)
    _check_ws(ws, ws_bytes)
    _check(lib.ssm_forward(ctypes.byref(dims), ctypes.byref(layer), _ptr(x), _ptr(y), ctypes.byref(saved),
                           _ptr(ws), int(ws_bytes), _stream(stream)), "ssm_forward")


def ssm_adjoint_grad(dims: Dims, layer: Layer, x, saved: Saved, g, window: int, grads: Grads, ws,
                     ws_bytes: int, stream=None):
    import torch

    _need(x, "x", dims.T * dims.P, _io(dims))
    _need(g, "g", dims.T * dims.P, torch.float32)
    _check_ws(ws, ws_bytes)
    _check(lib.ssm_adjoint_grad(ctypes.byref(dims), ctypes.byref(layer), _ptr(x), ctypes.byref(saved), _ptr(g),
                                int(window), ctypes.byref(grads), _ptr(ws), int(ws_bytes), _stream(stream)),
           "ssm_adjoint_grad")


NOALLOC_SCRATCH_BYTES = 256 << 20  # SSM_NOALLOC_SCRATCH_BYTES of the C header


def ssm_adjoint_grad_noalloc(dims: Dims, layer: Layer, x, saved: Saved, g, window: int, grads: Grads,
                             stream=None):
    """ssm_adjoint_grad with the library's own device array as workspace."""
    import torch

    _need(x, "x", dims.T * dims.P, _io(dims))
    _need(g, "g", dims.T * dims.P, torch.float32)
    _check(lib.ssm_adjoint_grad_noalloc(ctypes.byref(dims), ctypes.byref(layer), _ptr(x), ctypes.byref(saved),
                                        _ptr(g), int(window), ctypes.byref(grads), _stream(stream)),
           "ssm_adjoint_grad_noalloc")


def _event_array(events):
    """torch.cuda.Event objects (or None) -> C array of hipEvent_t handles."""
    arr = (ctypes.c_void_p * len(events))()
    for i, ev in enumerate(events):
        arr[i] = None if ev is None else int(ev.cuda_event)
    return arr


def ssm_forward_timed(dims: Dims, layer: Layer, x, y, saved: Saved, ws, ws_bytes: int, events, stream=None):
    import torch

    _need(x, "x", dims.T * dims.P, _io(dims))
    _need(y, "y", dims.T * dims.P, torch.float32)
    _check_ws(ws, ws_bytes)
    arr = _event_array(events)
    _check(lib.ssm_forward_timed(ctypes.byref(dims), ctypes.byref(layer), _ptr(x), _ptr(y), ctypes.byref(saved),
                                 _ptr(ws), int(ws_bytes), _stream(stream), arr, len(events)),
           "ssm_forward_timed")


def ssm_adjoint_grad_timed(dims: Dims, layer: Layer, x, saved: Saved, g, window: int, grads: Grads, ws,
                           ws_bytes: int, events, stream=None):
    """events: [0..6] phase marks, then two per slab around the fused reverse
    kernel's launches (see the C header)."""
    import torch

    _need(x, "x", dims.T * dims.P, _io(dims))
    _need(g, "g", dims.T * dims.P, torch.float32)
    _check_ws(ws, ws_bytes)
    arr = _event_array(events)
    _check(lib.ssm_adjoint_grad_timed(ctypes.byref(dims), ctypes.byref(layer), _ptr(x), ctypes.byref(saved),
                                      _ptr(g), int(window), ctypes.byref(grads), _ptr(ws), int(ws_bytes),
                                      _stream(stream), arr, len(events)),
           "ssm_adjoint_grad_timed")


def ssm_stack_grad(K: int, dims: Dims, layers, x0, g, window: int, grads, dx0, xK, ws, ws_bytes: int,
                   stream=None):
    import torch

    if len(layers) != K or len(grads) != K:
        raise SsmError(1, f"ssm_stack_grad: {len(layers)} layers and {len(grads)} gradient sets for K={K}")
    TP = dims.T * dims.P
    _need(x0, "x0", TP, _io(dims))
    _need(g, "g", TP, torch.float32)
    _need(dx0, "dx0", TP, torch.float32, optional=True)
    _need(xK, "xK", TP, torch.float32, optional=True)
    _check_ws(ws, ws_bytes)
    LArr = Layer * K
    GArr = Grads * K
    la = LArr(*layers)
    ga = GArr(*grads)
    _check(lib.ssm_stack_grad(int(K), ctypes.byref(dims), la, _ptr(x0), _ptr(g), int(window), ga, _ptr(dx0),
                              _ptr(xK), _ptr(ws), int(ws_bytes), _stream(stream)), "ssm_stack_grad")


# ---------------------------------------------------------------- torch-side conveniences

@dataclass
class LayerTensors:
    """Device tensors of one layer (io dtype for the weights)."""
    W_delta: object
    W_B: object
    W_C: object
    alpha: object
    delta_bias: object = None
    norm_scale: object = None  # [P] float32: stack layers that read the RMS-normalised stream

    def struct(self, dims: Dims) -> Layer:
        return layer_struct(dims, self.W_delta, self.W_B, self.W_C, self.alpha, self.delta_bias, self.norm_scale)


def io_dtype(io: str):
    import torch

    return torch.bfloat16 if io == "bf16" else torch.float32


def alloc_saved(dims: Dims, device="cuda", sub_states=False, all_states=False) -> dict:
    """Saved-state buffers; with sub_states, also the optional h_sub buffer
    (the forward then keeps the state of every 8th token for the gradient);
    with all_states, the h_all buffer of the store-everything baseline (the
    forward keeps every state)."""
    import torch

    K = (dims.T + dims.chunk - 1) // dims.chunk
    f = dict(device=device, dtype=torch.float32)
    out = {
        "s": torch.empty(dims.T, dims.P, **f),
        "b": torch.empty(dims.T, dims.N, **f),
        "c": torch.empty(dims.T, dims.N, **f),
        "h_ckpt": torch.empty(K, dims.P, dims.N, **f),
        "s_sum": torch.empty(K, dims.P, device=device, dtype=torch.float64),
    }
    if sub_states:
        nbytes = ssm_sub_state_bytes(dims)
        if nbytes == 0:
            raise SsmError(4, "ssm_sub_state_bytes")
        out["h_sub"] = torch.empty(nbytes // 4, **f)
    if all_states:
        nbytes = ssm_all_state_bytes(dims)
        if nbytes == 0:
            raise SsmError(4, "ssm_all_state_bytes")
        out["h_all"] = torch.empty(nbytes // 4, **f)
    return out


def alloc_workspace(nbytes: int, device="cuda"):
    import torch

    return torch.empty(max(int(nbytes), 1), device=device, dtype=torch.uint8)


def forward(dims: Dims, layer: LayerTensors, x, ws=None, saved=None, y=None, stream=None, sub_states=False,
            all_states=False):
    """Runs ssm_forward; returns (y, saved dict).  sub_states: keep h_sub;
    all_states: keep h_all, every state (when saved is not given)."""
    import torch

    nbytes = ssm_workspace_bytes(dims, 0, 0)
    if nbytes == 0:
        raise SsmError(4, "ssm_workspace_bytes")
    ws = alloc_workspace(nbytes, x.device) if ws is None else ws
    saved = alloc_saved(dims, x.device, sub_states, all_states) if saved is None else saved
    y = torch.empty(dims.T, dims.P, device=x.device, dtype=torch.float32) if y is None else y
    ssm_forward(dims, layer.struct(dims), x, y, saved_struct(saved, dims), ws, ws.numel(), stream)
    return y, saved


def alloc_grads(dims: Dims, want_dx=False, want_dalpha=True, want_dbias=True, device="cuda") -> dict:
    import torch

    f = dict(device=device, dtype=torch.float32)
    g = {"dW_delta": torch.empty(dims.P, dims.P, **f), "dW_B": torch.empty(dims.N, dims.P, **f),
         "dW_C": torch.empty(dims.N, dims.P, **f)}
    if want_dalpha:
        g["dalpha"] = torch.empty(dims.P, dims.N, **f)
    if want_dbias:
        g["dbias"] = torch.empty(dims.P, **f)
    if want_dx:
        g["dx"] = torch.empty(dims.T, dims.P, **f)
    return g


def adjoint_grad(dims: Dims, layer: LayerTensors, x, saved: dict, g, window: int, want_dx=False, ws=None,
                 grads=None, stream=None) -> dict:
    """Runs ssm_adjoint_grad; returns the gradient dict."""
    if saved.get("h_sub") is not None or saved.get("h_all") is not None:
        nbytes = ssm_grad_workspace_bytes_sub(dims, window)
    else:
        nbytes = ssm_workspace_bytes(dims, window, 0)
    if nbytes == 0:
        raise SsmError(4, "ssm_workspace_bytes")
    ws = alloc_workspace(nbytes, x.device) if ws is None else ws
    grads = alloc_grads(dims, want_dx=want_dx, device=x.device) if grads is None else grads
    ssm_adjoint_grad(dims, layer.struct(dims), x, saved_struct(saved, dims), g, window, grads_struct(grads, dims),
                     ws, ws.numel(), stream)
    return grads


def stack_grad(dims: Dims, layers: list, x0, g, window: int, ws=None, want_dx0=True, want_xK=True,
               stream=None):
    """Runs ssm_stack_grad; returns (list of gradient dicts, dx0, xK)."""
    import torch

    K = len(layers)
    structs = [lay.struct(dims) for lay in layers]
    nbytes = ssm_stack_workspace_bytes(K, dims, structs, window)
    if nbytes == 0:
        raise SsmError(4, "ssm_stack_workspace_bytes")
    ws = alloc_workspace(nbytes, x0.device) if ws is None else ws
    grads = [alloc_grads(dims, device=x0.device) for _ in range(K)]
    for gr, lay in zip(grads, layers):
        if lay.norm_scale is not None:
            gr["dnorm_scale"] = torch.empty(dims.P, device=x0.device, dtype=torch.float32)
    f = dict(device=x0.device, dtype=torch.float32)
    dx0 = torch.empty(dims.T, dims.P, **f) if want_dx0 else None
    xK = torch.empty(dims.T, dims.P, **f) if want_xK else None
    ssm_stack_grad(K, dims, structs, x0, g, window, [grads_struct(gr, dims) for gr in grads],
                   dx0, xK, ws, ws.numel(), stream)
    return grads, dx0, xK


# ---------------------------------------------------------------- unit probes (ssm_probe.h)

def ssm_probe_units(kind: int, wgs: int, iters: int, sink, clk, stream=None):
    """One probe launch (asynchronous): sink float32 [wgs * 256], clk int64
    [wgs * SSM_PROBE_WAVES_PER_WG * 4] (raw uint64 clock readings)."""
    import torch

    _need(sink, "sink", int(wgs) * 256, torch.float32)
    _need(clk, "clk", int(wgs) * SSM_PROBE_WAVES_PER_WG * 4, torch.int64)
    _check(lib.ssm_probe_units(int(kind), int(wgs), int(iters), _ptr(sink), _ptr(clk), _stream(stream)),
           "ssm_probe_units")


def ssm_probe_wall_clock_khz() -> int:
    khz = ctypes.c_int(0)
    _check(lib.ssm_probe_wall_clock_khz(ctypes.byref(khz)), "ssm_probe_wall_clock_khz")
    return int(khz.value)
