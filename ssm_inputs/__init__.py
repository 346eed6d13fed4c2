"""Seeded synthetic inputs for the selective-SSM gradient path.

This module is shared by the CPU oracle, the parity tests and the benchmark.
It only draws random numbers and rounds them to the storage dtype; it holds
none of the method's arithmetic (no projection, scan or gradient).

Shapes follow the pages' model (review of "Adjoint sharding for very long
context training of state space models", Section 3.1 as summarised under
"Assumptions"): x is [T][P] tokens by channels, W_delta is [P][P], W_B and
W_C are [N][P], alpha is [P][N], delta_bias is [P], g (the cotangent of y)
is [T][P].

Draw order (numpy PCG64, one generator per seed), all float32
standard normals unless stated:
    W_delta, W_B, W_C   (scaled by 1/sqrt(P))   -- repeated per layer for stacks
    u ~ U(1e-3, 1e-1) [P]                        -- only when bias="softplus_uniform"
    x [T][P], then g [T][P]                      -- drawn in row blocks
alpha[p, n] = n + 1.  x is multiplied by the case's x_scale (1 unless
stated) before rounding.  Inputs of io dtype bf16 are rounded from float32 by
round-to-nearest-even; g always stays float32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "LayerCase",
    "CASES",
    "bf16_round",
    "make_layer",
    "make_stack",
    "window_pin_case",
]


@dataclasses.dataclass(frozen=True)
class LayerCase:
    """One synthetic workload.

    io     : "f32" or "bf16" -- storage dtype of x and the weights.
    bias   : "zero"              -> delta_bias = 0
             "softplus_uniform"  -> softplus(delta_bias) ~ U(1e-3, 1e-1)
             "softplus_values"   -> softplus(delta_bias) cycles through `bias_u`
    wdelta : "normal" (W ~ N(0, 1/P)) or "zero" (W_delta = 0; then softplus(Delta)
             equals softplus(delta_bias) exactly).
    x_scale: standard deviation of x (x = x_scale * N(0, 1)).  The 4-layer
             N=64 stack uses 1/sqrt(N): a layer's output is cubic in its input
             (b, x and c are each linear in it), and with unit-variance x the
             residual stream of that stack passes the float32 range by the
             third layer.
    """

    name: str
    T: int
    P: int
    N: int
    io: str = "f32"
    windows: tuple = ()
    K: int = 1
    bias: str = "zero"
    bias_u: tuple = ()
    wdelta: str = "normal"
    seed: int = 0
    x_scale: float = 1.0


# The five workloads of the hot path (sizes from the method's problem
# statement: one layer at 16K / 128K / 1M tokens, and a 4-layer stack).
CASES = {
    0: LayerCase("layer_256tok_f32", 256, 16, 8, "f32", (256,), seed=0),
    1: LayerCase("layer_16k_f32", 16384, 1024, 16, "f32", (16384, 2048), seed=1),
    2: LayerCase("layer_128k_bf16", 131072, 2048, 16, "bf16", (1024, 8192), seed=2),
    3: LayerCase("layer_1m_bf16", 1048576, 2048, 16, "bf16", (4096,),
                 bias="softplus_uniform", seed=3),
    4: LayerCase("stack4_256k_bf16", 262144, 1536, 64, "bf16", (262144, 4096), K=4, seed=4,
                 x_scale=0.125),
}


def window_pin_case(seed: int = 100, T: int = 512, P: int = 8, N: int = 4) -> LayerCase:
    """Slow-decay case where adjacent windows give clearly different sums.

    W_delta = 0 so softplus(Delta_t[p]) = u_p exactly, with u_p spread over
    1e-3 .. 1e-1; alpha = n+1 keeps prod(a) close to 1 over hundreds of tokens.
    """
    return LayerCase(f"winpin_s{seed}", T, P, N, "f32", (), bias="softplus_values",
                     bias_u=(1e-3, 3e-3, 1e-2, 3e-2, 1e-1, 2e-3, 5e-3, 2e-2),
                     wdelta="zero", seed=seed)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # NaN stays NaN (not produced by these generators, kept for safety).
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def _normal_rows(rng: np.random.Generator, rows: int, cols: int, block: int = 1 << 14) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        out[r0:r1] = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
    return out


def _weights(rng: np.random.Generator, c: LayerCase) -> dict:
    scale = np.float32(1.0 / math.sqrt(c.P))
    wd = rng.standard_normal((c.P, c.P), dtype=np.float32) * scale
    wb = rng.standard_normal((c.N, c.P), dtype=np.float32) * scale
    wc = rng.standard_normal((c.N, c.P), dtype=np.float32) * scale
    if c.wdelta == "zero":
        wd = np.zeros_like(wd)
    if c.io == "bf16":
        wd, wb, wc = bf16_round(wd), bf16_round(wb), bf16_round(wc)
    return {"W_delta": wd, "W_B": wb, "W_C": wc}


def _bias(rng: np.random.Generator, c: LayerCase) -> np.ndarray:
    if c.bias == "zero":
        return np.zeros(c.P, dtype=np.float32)
    if c.bias == "softplus_uniform":
        u = rng.uniform(1e-3, 1e-1, size=c.P)
    elif c.bias == "softplus_values":
        vals = np.asarray(c.bias_u, dtype=np.float64)
        u = vals[np.arange(c.P) % len(vals)]
    else:
        raise ValueError(c.bias)
    # inverse of softplus: the bias whose softplus is u
    return np.log(np.expm1(u)).astype(np.float32)


def _alpha(c: LayerCase) -> np.ndarray:
    return np.tile(np.arange(1, c.N + 1, dtype=np.float32), (c.P, 1))


def make_layer(c: LayerCase, T: int | None = None) -> dict:
    """Inputs of one layer: float32 numpy arrays (bf16-valued where io == bf16).

    T overrides the token count (a prefix of the same draw order is *not*
    implied: x and g are drawn at the requested T).
    """
    T = c.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(c.seed))
    d = _weights(rng, c)
    d["delta_bias"] = _bias(rng, c)
    x = _normal_rows(rng, T, c.P)
    if c.x_scale != 1.0:
        x *= np.float32(c.x_scale)
    if c.io == "bf16":
        x = bf16_round(x)
    g = _normal_rows(rng, T, c.P)
    d.update(x=x, g=g, alpha=_alpha(c), T=T, P=c.P, N=c.N, io=c.io)
    return d


def make_stack(c: LayerCase, K: int | None = None, T: int | None = None) -> dict:
    """Inputs of a K-layer residual stack: per-layer weights, then x0 and g."""
    K = c.K if K is None else K
    T = c.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(c.seed))
    layers = []
    for _ in range(K):
        w = _weights(rng, c)
        w["delta_bias"] = np.zeros(c.P, dtype=np.float32)
        w["alpha"] = _alpha(c)
        layers.append(w)
    x = _normal_rows(rng, T, c.P)
    if c.x_scale != 1.0:
        x *= np.float32(c.x_scale)
    if c.io == "bf16":
        x = bf16_round(x)
    g = _normal_rows(rng, T, c.P)
    return {"layers": layers, "x": x, "g": g, "T": T, "P": c.P, "N": c.N, "K": K, "io": c.io}


def make_layer_device(c: LayerCase, device="cuda", T: int | None = None) -> dict:
    """Large workloads: weights, bias and alpha from the numpy stream above
    (same draws as make_layer), x and g drawn on the device with torch's
    seeded Philox generator (standard normal float32, x then g; x rounded to
    bfloat16 by round-to-nearest-even when io == bf16).  Returns torch
    tensors on `device` plus the numpy weights."""
    import torch

    T = c.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(c.seed))
    d = _weights(rng, c)
    d["delta_bias"] = _bias(rng, c)
    d["alpha"] = _alpha(c)
    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_003 * (c.seed + 1))
    x = torch.randn(T, c.P, generator=gen, device=device, dtype=torch.float32)
    if c.x_scale != 1.0:
        x *= c.x_scale
    if c.io == "bf16":
        x = x.to(torch.bfloat16)
    g = torch.randn(T, c.P, generator=gen, device=device, dtype=torch.float32)
    d.update(x_dev=x, g_dev=g, T=T, P=c.P, N=c.N, io=c.io)
    return d


def small_case(T: int, P: int, N: int, seed: int, io: str = "f32", bias: str = "zero",
               wdelta: str = "normal") -> LayerCase:
    """Ad-hoc small case with the same distributions (tests of edge shapes)."""
    return LayerCase(f"small_T{T}_P{P}_N{N}_s{seed}", T, P, N, io, (), bias=bias,
                     wdelta=wdelta, seed=seed)
