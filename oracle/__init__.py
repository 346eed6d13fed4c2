"""fp64 CPU oracle of the selective-SSM gradient path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library or its binding.  It
shares no code with the GPU path; the only common import is the seeded input
generator (ssm_inputs), which contains none of the method's arithmetic.

The arithmetic lives in ssm_oracle.c (plain loops in double precision); this
module builds it with gcc, loads it with ctypes and composes the steps:

  projections  Delta = W_delta x + bias, b = W_B x, c = W_C x
  forward      h_t = a_t h_{t-1} + b_t x_t, y_t = sum_n c_t h_t
               (review of "Adjoint sharding for very long context training of
               state space models", Assumptions / Section 3.1)
  adjoint sums mu (Proposition 1 reverse recurrence, the windowed identity, or
               the literal Proposition 2 double sum, "Core claim")
  local VJPs   dDelta, dalpha, dbias, db, dc, direct dx
  time sums    dW = sum_t (per-token cotangent) x_t^T, dx through W
  stack        residual layers r^{k+1} = r^k + y^k(cast(r^k)), loss on r^K,
               each layer driven by the total cotangent of its output
               (Proposition 3, "Core claim"; the cotangent reading is recorded
               in the design notes); optionally the layer input is the
               normalised stream cast(RMSNorm_gamma(r^k)) (the review's
               Algorithm 1 normalised input; the norm is a reading)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc_ssm.so")
_lib = None

BPTT, WINDOW_IDENTITY, LITERAL = 0, 1, 2

_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_project.argtypes = [_i64, _i64, _i64, _d, _d, _d, _d]
    lib.orc_project.restype = None
    lib.orc_forward.argtypes = [_i64, _i64, _i64, _d, _d, _d, _d, _d, _d, _i64, _d]
    lib.orc_forward.restype = None
    lib.orc_layer_grad.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _d, _d, _d, _d, _d, _d,
                                   _d, _d, _d, _d, _d, _d, _d]
    lib.orc_layer_grad.restype = ctypes.c_int
    lib.orc_weight_grad.argtypes = [_i64, _i64, _i64, _d, _d, _d]
    lib.orc_weight_grad.restype = None
    lib.orc_input_grad.argtypes = [_i64, _i64, _i64, _d, _d, _d]
    lib.orc_input_grad.restype = None
    lib.orc_cast_input.argtypes = [_i64, _d, ctypes.c_int, _d]
    lib.orc_cast_input.restype = None
    lib.orc_rmsnorm.argtypes = [_i64, _i64, _d, _d, ctypes.c_double, _d, _d]
    lib.orc_rmsnorm.restype = None
    lib.orc_rmsnorm_vjp.argtypes = [_i64, _i64, _d, _d, ctypes.c_double, _d, _d, _d]
    lib.orc_rmsnorm_vjp.restype = None
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    return _load().orc_num_threads()


def _pd(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_d)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def project(x: np.ndarray, W: np.ndarray, bias: np.ndarray | None = None,
            block: int = 1 << 14, blas: bool = False) -> np.ndarray:
    """out[t][m] = sum_q W[m][q] x[t][q] (+ bias[m]), float64 (row blocks of x).

    blas: each row block's product by numpy's float64 matmul (a library
    routine for the same sum, in its own summation order) instead of the
    plain C loops -- for the million-token workloads."""
    W = _f64(W)
    T, P = x.shape
    M = W.shape[0]
    out = np.empty((T, M), dtype=np.float64)
    bias64 = _f64(bias) if bias is not None else None
    if blas:
        Wt = np.ascontiguousarray(W.T)
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            np.matmul(_f64(x[t0:t1]), Wt, out=out[t0:t1])
            if bias64 is not None:
                out[t0:t1] += bias64
        return out
    bptr = _pd(bias64) if bias64 is not None else ctypes.cast(None, _d)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        xb = _f64(x[t0:t1])
        ob = np.empty((t1 - t0, M), dtype=np.float64)
        _load().orc_project(t1 - t0, P, M, _pd(xb), _pd(W), bptr, _pd(ob))
        out[t0:t1] = ob
    return out


def projections(inp: dict, x: np.ndarray | None = None, chans=None, blas: bool = False) -> dict:
    """Delta (for `chans`, default all), b and c of one layer."""
    x = inp["x"] if x is None else x
    Wd = np.asarray(inp["W_delta"])
    bias = np.asarray(inp["delta_bias"])
    if chans is not None:
        chans = np.asarray(chans, dtype=np.int64)
        Wd = Wd[chans]
        bias = bias[chans]
    return {
        "delta": project(x, Wd, bias, blas=blas),
        "b": project(x, inp["W_B"], blas=blas),
        "c": project(x, inp["W_C"], blas=blas),
    }


def forward(inp: dict, C: int = 0, x: np.ndarray | None = None) -> dict:
    """y [T][P] (float64) and, if C > 0, h_{kC-1} checkpoints [ceil(T/C)][P][N]."""
    x = _f64(inp["x"] if x is None else x)
    T, P = x.shape
    N = inp["W_B"].shape[0]
    pr = projections(inp, x=x)
    y = np.empty((T, P), dtype=np.float64)
    nck = (T + C - 1) // C if C > 0 else 0
    hck = np.zeros((max(nck, 1), P, N), dtype=np.float64)
    _load().orc_forward(T, P, N, _pd(pr["delta"]), _pd(pr["b"]), _pd(pr["c"]), _pd(x),
                        _pd(_f64(inp["alpha"])), _pd(y), C, _pd(hck))
    out = dict(pr)
    out["y"] = y
    if C > 0:
        out["h_ckpt"] = hck[:nck]
    return out


def loss(inp: dict, x: np.ndarray | None = None, g: np.ndarray | None = None) -> float:
    """L = sum_t <g_t, y_t> (float64)."""
    y = forward(inp, x=x)["y"]
    g = _f64(inp["g"] if g is None else g)
    return float(np.sum(g * y))


def _mode_for(window: int, T: int, method: str) -> int:
    if method == "literal":
        return LITERAL
    if method == "identity":
        return WINDOW_IDENTITY
    if method == "bptt":
        return BPTT
    if method == "auto":
        return BPTT if window >= T else WINDOW_IDENTITY
    raise ValueError(method)


def layer_grad(inp: dict, window: int | None = None, method: str = "auto",
               x: np.ndarray | None = None, g: np.ndarray | None = None,
               want_dx: bool = True) -> dict:
    """All gradients of one layer for loss sum_t <g_t, y_t> (window None = exact).

    Returns float64 arrays: y, delta, b, c, dDelta, db, dc, dxdir, dW_delta,
    dW_B, dW_C, dalpha, dbias and (want_dx) dx.
    """
    x = _f64(inp["x"] if x is None else x)
    g = _f64(inp["g"] if g is None else g)
    T, P = x.shape
    N = inp["W_B"].shape[0]
    W = T if window is None else int(window)
    mode = _mode_for(W, T, method)
    pr = projections(inp, x=x)
    y = np.empty((T, P))
    dD = np.empty((T, P))
    dxd = np.empty((T, P))
    dal = np.empty((P, N))
    dbi = np.empty(P)
    db = np.empty((T, N))
    dc = np.empty((T, N))
    rc = _load().orc_layer_grad(T, P, N, W, mode, _pd(pr["delta"]), _pd(pr["b"]), _pd(pr["c"]),
                                _pd(x), _pd(g), _pd(_f64(inp["alpha"])), _pd(y), _pd(dD), _pd(dxd),
                                _pd(dal), _pd(dbi), _pd(db), _pd(dc))
    if rc != 0:
        raise RuntimeError("oracle layer_grad failed (mode/window/allocation)")
    lib = _load()
    dWd = np.empty((P, P))
    dWb = np.empty((N, P))
    dWc = np.empty((N, P))
    lib.orc_weight_grad(T, P, P, _pd(dD), _pd(x), _pd(dWd))
    lib.orc_weight_grad(T, P, N, _pd(db), _pd(x), _pd(dWb))
    lib.orc_weight_grad(T, P, N, _pd(dc), _pd(x), _pd(dWc))
    out = dict(pr)
    out.update(y=y, dDelta=dD, dxdir=dxd, dalpha=dal, dbias=dbi, db=db, dc=dc,
               dW_delta=dWd, dW_B=dWb, dW_C=dWc)
    if want_dx:
        dx = dxd.copy()
        lib.orc_input_grad(T, P, P, _pd(dD), _pd(_f64(inp["W_delta"])), _pd(dx))
        lib.orc_input_grad(T, P, N, _pd(db), _pd(_f64(inp["W_B"])), _pd(dx))
        lib.orc_input_grad(T, P, N, _pd(dc), _pd(_f64(inp["W_C"])), _pd(dx))
        out["dx"] = dx
    return out


def channel_grad(inp: dict, chans, window: int | None = None, method: str = "auto",
                 g_cols: np.ndarray | None = None, blas: bool = False, bc: dict | None = None) -> dict:
    """Per-channel results for a subset of channels (large workloads).

    Channels are independent once b and c (which need every channel of x) are
    known, so Delta, y, dDelta, dxdir, dalpha, dbias and the dW_delta rows of
    the listed channels are exact; db and dc returned here are only the
    contributions of these channels.  g_cols, if given, is g restricted to
    the listed channels ([T][len(chans)]); otherwise inp["g"] is sliced.
    blas: projections and the dW_delta row sums by numpy's float64 matmul
    (see project).  bc: b and c of the layer when already known (they do
    not depend on the channel subset).
    """
    chans = np.asarray(chans, dtype=np.int64)
    x = inp["x"]
    T, P = x.shape
    N = inp["W_B"].shape[0]
    W = T if window is None else int(window)
    mode = _mode_for(W, T, method)
    if bc is None:
        pr = projections(inp, x=x, chans=chans, blas=blas)
    else:
        pr = {"delta": project(x, np.asarray(inp["W_delta"])[chans], np.asarray(inp["delta_bias"])[chans],
                               blas=blas), "b": bc["b"], "c": bc["c"]}
    nc = len(chans)
    xc = _f64(x[:, chans])
    gc = _f64(np.asarray(inp["g"])[:, chans] if g_cols is None else g_cols)
    alc = _f64(np.asarray(inp["alpha"])[chans])
    y = np.empty((T, nc))
    dD = np.empty((T, nc))
    dxd = np.empty((T, nc))
    dal = np.empty((nc, N))
    dbi = np.empty(nc)
    db = np.empty((T, N))
    dc = np.empty((T, N))
    rc = _load().orc_layer_grad(T, nc, N, W, mode, _pd(pr["delta"]), _pd(pr["b"]), _pd(pr["c"]),
                                _pd(xc), _pd(gc), _pd(alc), _pd(y), _pd(dD), _pd(dxd), _pd(dal),
                                _pd(dbi), _pd(db), _pd(dc))
    if rc != 0:
        raise RuntimeError("oracle channel_grad failed")
    dWd_rows = np.zeros((nc, P))
    block = 1 << 14
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        if blas:
            dWd_rows += np.matmul(dD[t0:t1].T, _f64(x[t0:t1]))
            continue
        part = np.empty((nc, P))
        _load().orc_weight_grad(t1 - t0, P, nc, _pd(_f64(dD[t0:t1])), _pd(_f64(x[t0:t1])), _pd(part))
        dWd_rows += part
    return {"chans": chans, "delta": pr["delta"], "b": pr["b"], "c": pr["c"], "y": y,
            "dDelta": dD, "dxdir": dxd, "dalpha": dal, "dbias": dbi, "db_part": db,
            "dc_part": dc, "dW_delta_rows": dWd_rows}


def cast_input(r: np.ndarray, io: str) -> np.ndarray:
    """Layer-input cast of the residual stream: float64 -> float32 (-> bf16 RNE).

    io == "f64" keeps the stream in double (no cast; used by the pins).
    """
    r = _f64(r)
    if io == "f64":
        return r.copy()
    out = np.empty(r.shape, dtype=np.float64)
    _load().orc_cast_input(r.size, _pd(r), 1 if io == "bf16" else 0, _pd(out))
    return out


NORM_EPS = 1e-5  # epsilon of the RMS normalisation (part of its definition)


def rmsnorm(r: np.ndarray, gamma: np.ndarray, eps: float = NORM_EPS):
    """RMS normalisation of every row: (gamma * r / sqrt(mean(r^2) + eps), 1/rms)."""
    r = _f64(r)
    T, P = r.shape
    out = np.empty_like(r)
    rinv = np.empty(T, dtype=np.float64)
    g = _f64(gamma)
    _load().orc_rmsnorm(T, P, _pd(r), _pd(g), float(eps), _pd(out), _pd(rinv))
    return out, rinv


def rmsnorm_vjp(r: np.ndarray, gamma: np.ndarray, dout: np.ndarray, eps: float = NORM_EPS):
    """(dr, dgamma): the vector-Jacobian product of rmsnorm for cotangent dout."""
    r, g, d = _f64(r), _f64(gamma), _f64(dout)
    T, P = r.shape
    dr = np.empty_like(r)
    dg = np.empty(P, dtype=np.float64)
    _load().orc_rmsnorm_vjp(T, P, _pd(r), _pd(g), float(eps), _pd(d), _pd(dr), _pd(dg))
    return dr, dg


def stack_forward(st: dict) -> dict:
    """Residual stack: r^0 = x^0, x^k = cast(r^k) -- or cast(rmsnorm(r^k)) when
    the layer has a "norm_scale" -- and r^{k+1} = r^k + y^k."""
    r = _f64(st["x"])
    xs, ys, rs = [], [], []
    for lay in st["layers"]:
        rs.append(r)
        src = rmsnorm(r, lay["norm_scale"])[0] if lay.get("norm_scale") is not None else r
        xk = cast_input(src, st["io"])
        inp = dict(lay, x=xk, g=st["g"])
        yk = forward(inp, x=xk)["y"]
        xs.append(xk)
        ys.append(yk)
        r = r + yk
    return {"x_layers": xs, "y_layers": ys, "r_layers": rs, "r_final": r}


def stack_grad(st: dict, window: int | None = None) -> dict:
    """Gradients of L = sum <g, r^K> for every layer of the stack.

    Backward: delta = g; for k = K-1..0 run the layer gradient with cotangent
    delta on y^k (the layer's parameters see the total derivative of the loss
    with respect to their output), then delta += dx^k, or the normalisation's
    VJP of dx^k when the layer normalises its input (the cast is treated as
    the identity).  Returns per-layer gradient dicts, dx0 and the forward.
    """
    fw = stack_forward(st)
    K = len(st["layers"])
    delta = _f64(st["g"])
    grads = [None] * K
    for k in range(K - 1, -1, -1):
        lay = st["layers"][k]
        inp = dict(lay, x=fw["x_layers"][k], g=delta)
        gk = layer_grad(inp, window=window, x=fw["x_layers"][k], g=delta, want_dx=True)
        grads[k] = gk
        if lay.get("norm_scale") is not None:
            dr, dg = rmsnorm_vjp(fw["r_layers"][k], lay["norm_scale"], gk["dx"])
            gk["dnorm_scale"] = dg
            delta = delta + dr
        else:
            delta = delta + gk["dx"]
    return {"layers": grads, "dx0": delta, "forward": fw}


def stack_loss(st: dict, x0: np.ndarray | None = None, layers=None) -> float:
    """sum <g, r^K> of the stack (float64)."""
    s = dict(st)
    if x0 is not None:
        s["x"] = x0
    if layers is not None:
        s["layers"] = layers
    r = stack_forward(s)["r_final"]
    return float(np.sum(_f64(st["g"]) * r))


if __name__ == "__main__":  # pragma: no cover - manual build helper
    print(build(force=True), file=sys.stderr)
