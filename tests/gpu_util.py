"""Helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the fp64 oracle on the same inputs."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return num if den == 0.0 else num / den


def p999_err(got, ref):
    """99.9th percentile of the elementwise |got - ref| / (|ref| + 1e-3 max|ref|),
    reported beside the per-tensor maximum (where elementwise relative errors
    near zeros are undefined, the 1e-3 max|ref| floor keeps them finite)."""
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if ref.size == 0:
        return 0.0
    floor = 1e-3 * float(np.max(np.abs(ref)))
    e = np.abs(got - ref) / (np.abs(ref) + floor) if floor > 0 else np.abs(got - ref)
    return float(np.percentile(e, 99.9))


def say(msg):
    print(msg, flush=True)


def to_dev(arr, io="f32"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if io == "bf16" else t


def layer_tensors(inp, io):
    import adjoint_gradients_amd as agm

    ns = inp.get("norm_scale")
    return agm.LayerTensors(to_dev(inp["W_delta"], io), to_dev(inp["W_B"], io), to_dev(inp["W_C"], io),
                            to_dev(inp["alpha"]), to_dev(inp["delta_bias"]),
                            None if ns is None else to_dev(np.asarray(ns, dtype=np.float32)))


def gpu_layer(inp, window, chunk, want_dx=True, io=None, g=None, sub_states=False, all_states=False):
    """Forward + adjoint gradient of one layer on the GPU; returns numpy float64 dict.
    sub_states: the forward keeps the sub-chunk states (saved h_sub) for the gradient;
    all_states: it keeps every state (saved h_all, the store-everything baseline)."""
    import torch

    import adjoint_gradients_amd as agm

    io = io or inp["io"]
    T, P = inp["x"].shape
    N = inp["W_B"].shape[0]
    dims = agm.make_dims(T, P, N, chunk, io)
    lay = layer_tensors(inp, io)
    x = to_dev(inp["x"], io)
    gg = to_dev(inp["g"] if g is None else g)
    y, saved = agm.forward(dims, lay, x, sub_states=sub_states, all_states=all_states)
    grads = agm.adjoint_grad(dims, lay, x, saved, gg, window, want_dx=want_dx)
    torch.cuda.synchronize()
    out = {k: v.double().cpu().numpy() for k, v in grads.items()}
    out["y"] = y.double().cpu().numpy()
    for k, v in saved.items():
        if k not in ("h_sub", "h_all"):  # private layouts
            out["saved_" + k] = v.double().cpu().numpy()
    return out


def oracle_inputs(inp):
    """float64 copies of the (exact) float32 / bf16-valued inputs."""
    return {k: (np.asarray(v, dtype=np.float64) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}


def compare(got, ref, keys, tol, label=""):
    errs = {}
    for gk, rk in keys:
        errs[gk] = rel_err(got[gk], ref[rk])
    p = {gk: p999_err(got[gk], ref[rk]) for gk, rk in keys}
    worst = max(p, key=p.get) if p else None
    say(f"[{label}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items())
        + (f" | elementwise p99.9 worst {worst}={p[worst]:.2e}" if worst else ""))
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"{label}: over tolerance {tol}: {bad}"
    return errs


GRAD_KEYS = [("dW_delta", "dW_delta"), ("dW_B", "dW_B"), ("dW_C", "dW_C"), ("dalpha", "dalpha"),
             ("dbias", "dbias"), ("dx", "dx"), ("y", "y")]
