#!/usr/bin/env python3
"""Throughput of the selective-SSM adjoint-gradient hot path on one MI355X.

One step = ssm_forward (projection GEMM, chunked forward scan with h
checkpoints, y) + ssm_adjoint_grad (windowed reverse adjoint scan fused with
the local VJPs, channel/chunk reductions, weight-gradient GEMM) on a
1,048,576-token, 2048-channel, N=16 layer with bf16 x and weights, fp32
state, window 4096 and h stored only at the 256-token chunk boundaries (the
gradient rebuilds the states inside each chunk).  Inputs are synthetic,
seeded and resident in HBM before the timed region.  Prints one JSON line.
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOADS = {
    # name: (index in ssm_inputs.CASES, window, chunk, states the forward keeps besides the chunk
    # checkpoints: None, "sub" (every 8th token's) or "all" (every token's: the store-everything
    # backpropagation baseline))
    "layer1m": (3, 4096, 256, None),         # 1M tokens, P = 2048, N = 16, bf16, chunk checkpoints only
    "layer1m_substates": (3, 4096, 256, "sub"),
    "layer1m_bptt": (3, 4096, 256, "all"),   # store-everything baseline: 128 GiB of states
    "layer1m_exact": (3, 1048576, 256, None),
    "layer1m_bptt_exact": (3, 1048576, 256, "all"),
    "layer128k": (2, 8192, 256, None),       # 128K tokens, P = 2048, N = 16, bf16
    "layer128k_w1k": (2, 1024, 256, None),
    "layer128k_bptt": (2, 8192, 256, "all"),
    "layer16k": (1, 2048, 256, None),        # 16K tokens, P = 1024, N = 16, fp32
    "layer16k_exact": (1, 16384, 256, None),
    "stack4": (4, 4096, 256, None),  # the 4-layer residual stack (ssm_stack_grad), timed whole
    "stack4_norm": (4, 4096, 256, None),  # the same stack, every layer reading the RMS-normalised stream
}

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16
MFMA_F32_PEAK_TFS = 157.3
# VALU issue rate without packed-fp32 forms: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz
VALU_PEAK_GOPS = 256 * 4 * 16 * 2.4

FWD_PHASES = ["proj_gemm", "fwd_local", "fwd_carry", "fwd_final"]
# Between the carry and reduction marks the gradient alternates, slab by slab
# of chunks, bwd_slab_prep (the rebuild of the slab's sub-chunk states, and,
# when the forward kept none, the slab's chunk aggregates, window composition
# and carry, formed in the same pass) with bwd_main (the fused reverse kernel).
BWD_PHASES = ["bwd_local", "bwd_carry", "bwd_slab_prep", "bwd_main", "bwd_reduce", "wgrad_gemm", "dx_gemm"]


def algorithmic(name, T, P, N, C, W, s_io, kept=None, _prep=False):
    """Per-launch algorithmic work of a phase: (bytes, flops, valu_ops).

    Bytes count each compulsory HBM stream once.  With kept == "sub" the
    forward keeps the state entering every 8th token (T/8 x P x N fp32), with
    kept == "all" every state (T x P x N fp32, the store-everything
    baseline): the final forward scan writes them and the fused gradient
    kernel reads them.  valu_ops counts the VALU
    issue slots of the method's own arithmetic per (t, p, n) element, a
    hardware exp2 counting 2 (it issues at half rate on gfx950):
      a_t = exp(-alpha s_t)                          mul + exp        3
      h_t = a_t h_{t-1} + b_t x_t                    mul + fma        2
      y_t += c_t h_t                                 fma              1
      mu_i = a_{i+1} mu_{i+1} + g_i c_i              mul + fma        2
      window term - g_{i+W} c_{i+W} D_i,
        D_i = exp(-alpha (S_{i+W} - S_i))            mul + exp + mul + fma   5
      da = mu h_{i-1}; da a; dDelta and dalpha sums  mul, mul, fma, fma      4
      db = sum_p mu x ; dc = sum_p g h               (mul + add) x 2         4
      dx_dir = sum_n mu b                            fma              1
    Per-(t, p) work (softplus, sigma, the dDelta scale) is amortised over N
    and left out."""
    E = T * P * N
    K = (T + C - 1) // C
    win = W < T
    if name == "proj_gemm":
        return (T * (P * s_io + 4 * P + 8 * N), 2.0 * T * P * (P + 2 * N), 0)
    if name == "fwd_local":
        return (T * (P * s_io + 4 * P + 4 * N) + K * P * N * 12, 0, 5 * E)
    if name == "fwd_carry":
        return (K * P * N * 8 + K * P * 8, 0, 4 * K * P * N)
    sub = {"sub": (T + 7) // 8 * P * N * 4, "all": T * P * N * 4}.get(kept, 0)
    if name == "fwd_final":
        return (T * (P * s_io + 8 * P + 8 * N) + K * P * N * 4 + sub, 0, 6 * E)
    # a window of whole chunks is composed from exact chunk aggregates in the
    # carry pass, so the local pass then walks no window term
    compose = win and W % C == 0
    # without states kept by the forward, exact local aggregates (N a
    # multiple of 4: the rebuild stages the chunk rows, in parts if need be)
    # are formed slab by slab in the rebuild walk (phase bwd_slab_prep), with
    # the composition and carry
    fused = kept is None and (not win or compose) and N % 4 == 0
    if name in ("bwd_local", "bwd_carry") and fused and not _prep:
        return (0, 0, 0)
    if name == "bwd_local":
        return (T * (8 * P + 4 * N) + K * P * N * 4, 0, (10 if win and not compose else 5) * E)
    if name == "bwd_carry":
        return (K * P * N * 8 + K * P * 8, 0, (9 if compose else 4) * K * P * N)
    if name == "bwd_slab_prep":
        if kept is not None:
            return (0, 0, 0)
        # the local aggregates (bytes and slots as bwd_local) formed in the
        # forward walk that rebuilds the states -- the rebuild itself is
        # recompute, with no bytes or work of the method's own -- plus the
        # composition and the carry
        if not fused:
            return (0, 0, 0)
        lb, _, lo = algorithmic("bwd_local", T, P, N, C, W, s_io, None, True)
        cb, _, co = algorithmic("bwd_carry", T, P, N, C, W, s_io, None, True)
        return (lb + cb, 0, lo + co)
    if name == "bwd_main":
        # per token: x, s, g, b, c, dDelta (io) and db/dc, plus h_ckpt once per chunk
        return (T * (P * s_io + 4 * P + 4 * P + 8 * N + P * s_io + 8 * N) + K * P * N * 4 + sub, 0,
                (21 if win else 16) * E)
    if name == "bwd_reduce":
        return (T * 2 * N * 4 * 2, 0, 0)
    if name == "wgrad_gemm":
        return (T * ((P + 2 * N) * s_io + P * s_io), 2.0 * T * P * (P + 2 * N), 0)
    if name == "dx_gemm":
        return (T * ((P + 2 * N) * s_io + 8 * P), 2.0 * T * P * (P + 2 * N), 0)
    return (0, 0, 0)


# Sources each phase's kernels are compiled from: a stored counter reading is
# only used while these files are byte-identical to when it was taken.
CSRC = os.path.join(ROOT, "adjoint_gradients_amd", "csrc")
PHASE_SOURCES = {
    "bwd_main": ["scan_bwd.hip", "bwd_main.inl", "red_layout.hpp", "ssm_common.hpp", "ssm_kernels.hpp"],
    "bwd_local": ["scan_bwd.hip", "bwd_main.inl", "red_layout.hpp", "ssm_common.hpp", "ssm_kernels.hpp"],
    "fwd_final": ["scan_fwd.hip", "ssm_common.hpp", "ssm_kernels.hpp"],
    "fwd_local": ["scan_fwd.hip", "ssm_common.hpp", "ssm_kernels.hpp"],
    "proj_gemm": ["gemm.hip", "gemm_dl.inl", "gemm_dl_index.hpp", "gemm_bf16.inl", "ssm_kernels.hpp"],
    "wgrad_gemm": ["gemm.hip", "gemm_dl.inl", "gemm_dl_index.hpp", "gemm_bf16.inl", "ssm_kernels.hpp"],
}


# C/C++ tokens that matter for the hash: string and character literals are
# kept whole, comments dropped, runs of whitespace folded to one space.
_SRC_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/|\s+', re.S)


def code_only(text):
    """Source text without comments and with whitespace folded, so that an
    edit of comments or layout alone does not change the hash below."""
    def sub(m):
        t = m.group(0)
        if t.startswith("//") or t.startswith("/*"):
            return " "
        if t[0].isspace():
            return " "
        return t
    return re.sub(r" +", " ", _SRC_TOKENS.sub(sub, text)).strip()


def source_hash(phase):
    """Hash of the code (comments and whitespace aside) of the sources a
    phase's kernels are built from."""
    import hashlib

    h = hashlib.sha256()
    for f in PHASE_SOURCES.get(phase, []):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(phase, workload):
    """HBM bytes per launch from profiles/traffic_<phase>_<workload>.md (FETCH_SIZE
    and WRITE_SIZE, calibrated against a plain copy), or None when there is no
    such summary or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{phase}_{workload}.md")
    if phase not in PHASE_SOURCES or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^- (\w+): `?([^`\s]+)`?", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("source_sha256") != source_hash(phase):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HipEvents:
    """Raw hipEvent_t handles (created through the HIP runtime) for the
    library's phase marks; torch's Event objects cannot see records made
    outside torch."""

    def __init__(self):
        import ctypes

        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.all = []

    def make(self, n):
        out = []
        for _ in range(n):
            h = self.ct.c_void_p()
            rc = self.hip.hipEventCreate(self.ct.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            out.append(_RawEvent(h.value))
            self.all.append(h.value)
        return out

    def ms(self, a, b):
        f = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(f), self.ct.c_void_p(a.cuda_event),
                                          self.ct.c_void_p(b.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(f.value)

    def destroy(self):
        for h in self.all:
            self.hip.hipEventDestroy(self.ct.c_void_p(h))
        self.all = []


class _RawEvent:
    def __init__(self, handle):
        self.cuda_event = handle


def cpu_baseline(case, window, chunk, tokens):
    """Times the fp64 oracle (as it stands) on a token prefix of the workload."""
    import numpy as np

    import oracle
    from ssm_inputs import make_layer

    oracle.build(force=False)
    inp = make_layer(case, T=tokens)
    o = {k: (np.asarray(v, dtype=np.float64) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    t0 = time.perf_counter()
    oracle.layer_grad(o, window=window if window < tokens else None, want_dx=False)
    wall = time.perf_counter() - t0
    return {"value": tokens / wall, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"fp64 oracle forward+adjoint+VJP+weight grads on the first {tokens} of the "
                      f"{case.T} tokens of the {case.name} workload (P={case.P}, N={case.N}, window={window}); "
                      f"wall {wall:.2f} s; value = that prefix's tokens / wall (the oracle's cost is linear "
                      f"in T at a fixed window)"}


def study_truncation():
    """Truncation quality: relative gradient error of the W-token adjoint window
    against the exact adjoint (W = T), for layers whose decay rate is set
    exactly: W_delta = 0, so softplus(Delta) = u in every channel and the decay
    rate of state n is u (n + 1).  The slowest state's tail beyond W weighs
    about exp(-u W).  fp32 throughout (the kernels' own rounding is ~1e-6)."""
    import math

    import torch

    import adjoint_gradients_amd as agm
    from ssm_inputs import LayerCase, make_layer

    T, P, N, C = 32768, 256, 16, 256
    keys = ("dW_delta", "dW_B", "dW_C", "dalpha", "dbias", "dx")
    rows = []
    for u in (1e-4, 1e-3, 1e-2, 1e-1):
        case = LayerCase(f"trunc_u{u:g}", T, P, N, "f32", (), bias="softplus_values", bias_u=(u,),
                         wdelta="zero", seed=7)
        inp = make_layer(case)
        dev = "cuda:0"
        t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
        lay = agm.LayerTensors(t(inp["W_delta"]), t(inp["W_B"]), t(inp["W_C"]), t(inp["alpha"]),
                               t(inp["delta_bias"]))
        x, g = t(inp["x"]), t(inp["g"])
        dims = agm.make_dims(T, P, N, C, "f32")
        _, saved = agm.forward(dims, lay, x)
        ref = agm.adjoint_grad(dims, lay, x, saved, g, T, want_dx=True)
        for W in (16, 64, 256, 1024, 4096):
            gr = agm.adjoint_grad(dims, lay, x, saved, g, W, want_dx=True)
            err = {k: float((gr[k].double() - ref[k].double()).norm() / ref[k].double().norm()) for k in keys}
            row = {"study": "truncation", "T": T, "P": P, "N": N, "u": u, "W": W,
                   "tail_exp_minus_uW": math.exp(-u * W), "rel_err": err}
            rows.append(row)
            print(json.dumps(row), flush=True)
    print(f"{'u':>8s} {'W':>6s} {'exp(-uW)':>10s} " + " ".join(f"{k:>9s}" for k in keys), file=sys.stderr)
    for r in rows:
        print(f"{r['u']:8.0e} {r['W']:6d} {r['tail_exp_minus_uW']:10.2e} "
              + " ".join(f"{r['rel_err'][k]:9.2e}" for k in keys), file=sys.stderr)


def study_memory():
    """Device memory and time of one layer's forward + gradient at the 128K and
    1M-token workloads, for the three kinds of kept state: chunk checkpoints
    only (the adjoint path as benchmarked), also every 8th token's state, and
    every state (the store-everything backpropagation baseline).  The library
    allocates nothing, so the memory is the caller's buffers: torch's peak of
    allocated bytes over both calls.  Beside them, the per-token storage of
    the reviewed paper's memory analysis ({A_t, C_t, h_t, y_t} for every token)
    applied to this layer in fp16, T (2 P N + N + P) x 2 bytes."""
    import torch

    import adjoint_gradients_amd as agm
    from ssm_inputs import CASES, make_layer_device

    gib = float(1 << 30)
    for case_idx, window in ((2, 1024), (3, 4096)):
        case = CASES[case_idx]
        T, P, N, io = case.T, case.P, case.N, case.io
        dims = agm.make_dims(T, P, N, 256, io)
        for kept in (None, "sub", "all"):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            inp = make_layer_device(case, "cuda:0")
            dt = agm.io_dtype(io)
            dv = lambda a, d=torch.float32: torch.from_numpy(a).to("cuda:0").to(d)  # noqa: E731
            lay = agm.LayerTensors(dv(inp["W_delta"], dt), dv(inp["W_B"], dt), dv(inp["W_C"], dt),
                                   dv(inp["alpha"]), dv(inp["delta_bias"]))
            x, g = inp["x_dev"], inp["g_dev"]
            torch.cuda.synchronize()
            base = torch.cuda.memory_allocated()
            times = []
            for rep in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                y, saved = agm.forward(dims, lay, x, sub_states=kept == "sub", all_states=kept == "all")
                grads = agm.adjoint_grad(dims, lay, x, saved, g, window)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
                if rep < 2:
                    del y, saved, grads
            peak = torch.cuda.max_memory_allocated()
            row = {
                "study": "memory", "workload": case.name, "T": T, "P": P, "N": N, "window": window,
                "states_kept": {None: "chunk checkpoints", "sub": "every 8th token", "all": "every token"}[kept],
                "inputs_gib": round(base / gib, 3),
                "saved_gib": round(sum(v.numel() * v.element_size() for v in saved.values()) / gib, 3),
                "workspace_fwd_gib": round(agm.ssm_workspace_bytes(dims, 0, 0) / gib, 3),
                "workspace_grad_gib": round((agm.ssm_grad_workspace_bytes_sub(dims, window) if kept
                                             else agm.ssm_workspace_bytes(dims, window, 0)) / gib, 3),
                "peak_allocated_gib": round(peak / gib, 3),
                "ms_fwd_plus_grad_incl_allocation": round(min(times), 2),
                "paper_sec45_per_token_fp16_gib": round(T * (2 * P * N + N + P) * 2 / gib, 3),
            }
            print(json.dumps(row), flush=True)
            del y, saved, grads, inp, x, g, lay


# Unit probes: (name, kind, workgroups per CU, iterations, wave64 instructions
# of each kind per wavefront and iteration).  Eight waves per SIMD for the
# VALU probes, two for MFMA (as in the GEMMs); about 20-60 ms each.
UNIT_PROBES = (
    ("fp32_fma", 0, 8, 250000, {"fma": 8}),
    ("exp2", 1, 8, 125000, {"exp": 8}),
    ("exp2_and_fma", 2, 8, 100000, {"exp": 8, "fma": 8}),
    ("mfma_bf16_32x32x16", 3, 2, 150000, {"mfma": 4}),
)


def calibrate_units():
    """Issue rates of single gfx950 units (ssm_probe.h), each with the clock
    the chip ran that load at (shader-clock cycles over wall-clock time, read
    by every wavefront of the probe): the fp32 FMA rate, the cost of a
    v_exp_f32 in VALU issue cycles (the scans' roofline counts two slots), and
    the dense bf16 MFMA rate (the GEMMs' peak).  One JSON line per probe."""
    import torch

    import adjoint_gradients_amd as agm

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    khz = agm.ssm_probe_wall_clock_khz()
    for name, kind, per_cu, iters, counts in UNIT_PROBES:
        wgs = cus * per_cu
        waves = wgs * agm.SSM_PROBE_WAVES_PER_WG
        sink = torch.empty(wgs * 256, device="cuda:0", dtype=torch.float32)
        clk = torch.empty(waves * 4, device="cuda:0", dtype=torch.int64)
        agm.ssm_probe_units(kind, wgs, max(1, iters // 50), sink, clk)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        agm.ssm_probe_units(kind, wgs, iters, sink, clk)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        c = clk.view(waves, 4).cpu().double()
        ghz_w = (c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / (khz * 1e3)) / 1e9
        ghz = float(ghz_w.median())
        # SIMD issue cycles per wave64 instruction of the probe: 4 SIMDs a CU
        simd_cycles = 4.0 * cus * ghz * 1e9 * ms * 1e-3
        n_inst = waves * iters * sum(counts.values())
        rec = {"probe": name, "workgroups": wgs, "waves_per_simd": per_cu * agm.SSM_PROBE_WAVES_PER_WG // 4,
               "iters": iters, "ms": round(ms, 3), "clock_ghz": round(ghz, 3),
               "clock_ghz_min_max": [round(float(ghz_w.min()), 3), round(float(ghz_w.max()), 3)],
               "simd_cycles_per_wave_instruction": round(simd_cycles / n_inst, 3)}
        if "mfma" in counts:
            flops = waves * iters * counts["mfma"] * 2 * 32 * 32 * 16
            rec["tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
            rec["flops_per_cu_per_clock"] = round(flops / (ms * 1e-3) / cus / (ghz * 1e9), 1)
            rec["published_peak_at_this_clock_tflops"] = round(MFMA_BF16_PEAK_TFS * ghz / 2.4, 1)
        else:
            lane_ops = waves * 64 * iters * sum(counts.values())
            rec["lane_ops_per_s"] = float(f"{lane_ops / (ms * 1e-3):.4g}")
            rec["lane_ops_per_cu_per_clock"] = round(lane_ops / (ms * 1e-3) / cus / (ghz * 1e9), 2)
            if kind == 2:
                # one exp and one FMA a pair: the exp's issue cycles beyond the FMA's 4
                rec["exp_issue_slots_when_mixed"] = round((2 * simd_cycles / n_inst - 4.0) / 4.0, 2)
        print(json.dumps(rec), flush=True)


def bench_stack(args, case_idx, window, chunk, norm=False):
    """One step of the K-layer residual stack: ssm_stack_grad (K forwards, then
    the K gradients in reverse with the cotangent passed down), timed whole
    with events on the library's stream.  Inputs as in the stack tests."""
    import numpy as np
    import torch

    import adjoint_gradients_amd as agm
    from ssm_inputs import CASES, _alpha, _weights

    case = CASES[case_idx]
    T, P, N, K = case.T, case.P, case.N, case.K
    dev = "cuda:0"
    torch.cuda.set_device(0)
    rng = np.random.Generator(np.random.PCG64(case.seed))
    nrng = np.random.default_rng(44)
    lays = []
    for _ in range(K):
        wts = _weights(rng, case)
        gam = None
        if norm:  # gamma ~ U(0.5, 1.5) at the stack's input scale 1 / sqrt(N)
            gam = torch.from_numpy((nrng.uniform(0.5, 1.5, P) / np.sqrt(N)).astype(np.float32)).to(dev)
        lays.append(agm.LayerTensors(*(torch.from_numpy(wts[k]).to(dev).to(torch.bfloat16)
                                       for k in ("W_delta", "W_B", "W_C")),
                                     torch.from_numpy(_alpha(case)).to(dev), torch.zeros(P, device=dev), gam))
    gen = torch.Generator(device=dev)
    gen.manual_seed(1_000_003 * (case.seed + 1))
    x0 = (torch.randn(T, P, generator=gen, device=dev) * case.x_scale).to(torch.bfloat16)
    g = torch.randn(T, P, generator=gen, device=dev)
    dims = agm.make_dims(T, P, N, chunk, "bf16")
    L = [lay.struct(dims) for lay in lays]
    ws = agm.alloc_workspace(agm.ssm_stack_workspace_bytes(K, dims, L, window), dev)
    grads = [agm.alloc_grads(dims, device=dev) for _ in range(K)]
    if norm:
        for gr in grads:
            gr["dnorm_scale"] = torch.empty(P, device=dev, dtype=torch.float32)
    dx0 = torch.empty(T, P, device=dev, dtype=torch.float32)
    xK = torch.empty(T, P, device=dev, dtype=torch.float32)
    G = [agm.grads_struct(gr, dims) for gr in grads]

    def step():
        agm.ssm_stack_grad(K, dims, L, x0, g, window, G, dx0, xK, ws, ws.numel())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    line = {
        "metric": "SSM adjoint-gradient tokens/s through a K-layer residual stack (fwd+adjoint+VJP)",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{case.name}: {K}-layer residual stack, T={T}, P={P}, N={N}, io=bf16, "
                               f"fp32 state and residual, window={window}, checkpoint every {chunk} tokens"
                               + (", RMS-normalised layer inputs" if norm else ""),
                   "T": T, "P": P, "N": N, "K": K, "window": window, "chunk": chunk, "normalised": norm},
        "roofline": None,
        "note": "stack call timed whole (no per-kernel events); the single-layer workloads carry the roofline",
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="layer1m", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=65536,
                    help="tokens of the workload the fp64 oracle is timed on (the CPU baseline sample)")
    ap.add_argument("--source-hash", metavar="PHASE", default=None,
                    help="print the hash of the sources a phase's kernels are built from and exit")
    ap.add_argument("--phases", action="store_true", help="print the per-phase breakdown to stderr")
    ap.add_argument("--study", choices=("truncation", "memory"), default=None,
                    help="run a measurement study instead of the benchmark (JSON lines on stdout)")
    ap.add_argument("--calibrate-units", action="store_true",
                    help="only run the unit probes (fp32 FMA, exp2, both, bf16 MFMA issue rates with the "
                         "clock the chip ran each at; JSON lines on stdout)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB three times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    args = ap.parse_args()
    if args.source_hash:
        print(source_hash(args.source_hash))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Sharded over time, each GPU would scan its own tokens and exchange one chunk aggregate per "
              "direction (a halo of W tokens for a truncated window) and all-reduce the weight gradients.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.study == "truncation":
        study_truncation()
        return
    if args.study == "memory":
        study_memory()
        return
    if args.calibrate_units:
        calibrate_units()
        return
    if args.calibrate_copy:
        # a plain device-to-device copy of known size: its FETCH_SIZE and
        # WRITE_SIZE counter readings calibrate the traffic figures, and its
        # event-timed rate is the copy bandwidth the HBM-bound kernels are
        # compared with (read + written bytes / time)
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, device="cuda:0", dtype=torch.float32)
        dst = torch.empty_like(src)
        ms = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3, "ms": [round(v, 4) for v in ms],
                          "copy_gbs_read_plus_write": round(2 * n * 4 / (min(ms) * 1e-3) / 1e9, 1)}), flush=True)
        return

    import adjoint_gradients_amd as agm
    from ssm_inputs import CASES, make_layer_device

    case_idx, window, chunk, kept = WORKLOADS[args.workload]
    if CASES[case_idx].K > 1:
        bench_stack(args, case_idx, window, chunk, norm=args.workload.endswith("norm"))
        return
    case = CASES[case_idx]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = make_layer_device(case, device=dev)
    T, P, N, io = case.T, case.P, case.N, case.io
    s_io = 2 if io == "bf16" else 4
    dt = torch.bfloat16 if io == "bf16" else torch.float32

    def dev_t(a, dtype=torch.float32):
        return torch.from_numpy(a).to(dev).to(dtype)

    lay = agm.LayerTensors(dev_t(inp["W_delta"], dt), dev_t(inp["W_B"], dt), dev_t(inp["W_C"], dt),
                           dev_t(inp["alpha"]), dev_t(inp["delta_bias"]))
    x, g = inp["x_dev"], inp["g_dev"]
    dims = agm.make_dims(T, P, N, chunk, io)
    ws_f = agm.alloc_workspace(agm.ssm_workspace_bytes(dims, 0, 0), dev)
    saved = agm.alloc_saved(dims, dev, sub_states=kept == "sub", all_states=kept == "all")
    ws_b = agm.alloc_workspace(agm.ssm_grad_workspace_bytes_sub(dims, window) if kept
                               else agm.ssm_workspace_bytes(dims, window, 0), dev)
    grads = agm.alloc_grads(dims, device=dev)
    y = torch.empty(T, P, device=dev, dtype=torch.float32)
    mem_total = torch.cuda.memory_allocated()  # everything the step uses, allocated before it runs
    L = lay.struct(dims)
    S = agm.saved_struct(saved, dims)
    G = agm.grads_struct(grads, dims)
    nslab = agm.ssm_grad_slab_count(dims, window, kept is not None)
    stream = torch.cuda.current_stream()

    hev = HipEvents()

    def new_events(n):
        return hev.make(n)

    def step(evf=None, evb=None):
        if evf is None:
            agm.ssm_forward(dims, L, x, y, S, ws_f, ws_f.numel())
            agm.ssm_adjoint_grad(dims, L, x, S, g, window, G, ws_b, ws_b.numel())
        else:
            agm.ssm_forward_timed(dims, L, x, y, S, ws_f, ws_f.numel(), evf)
            agm.ssm_adjoint_grad_timed(dims, L, x, S, g, window, G, ws_b, ws_b.numel(), evb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, phase events recorded on the library's stream
    evs = [(new_events(5), new_events(7 + 2 * nslab)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for evf, evb in evs:
        step(evf, evb)
    stop.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    # gradient marks: [0] start [1] local [2] carry [3] slabs done [4] reductions
    # [5] wgrad [6] dx, then [7 + 2 s], [8 + 2 s] around the fused kernel's launch
    # over slab s; the slab preparation passes fill the rest of [2]..[3]
    phase_ms = {k: 0.0 for k in FWD_PHASES + BWD_PHASES}
    marks = {"bwd_local": (0, 1), "bwd_carry": (1, 2), "bwd_reduce": (3, 4), "wgrad_gemm": (4, 5),
             "dx_gemm": (5, 6)}
    for evf, evb in evs:
        for i, k in enumerate(FWD_PHASES):
            phase_ms[k] += hev.ms(evf[i], evf[i + 1]) / args.steps
        for k, (i, j) in marks.items():
            phase_ms[k] += hev.ms(evb[i], evb[j]) / args.steps
        main = sum(hev.ms(evb[7 + 2 * q], evb[8 + 2 * q]) for q in range(nslab))
        phase_ms["bwd_main"] += main / args.steps
        phase_ms["bwd_slab_prep"] += (hev.ms(evb[2], evb[3]) - main) / args.steps
    hev.destroy()

    rows = []
    for k, ms in phase_ms.items():
        by, fl, ops = algorithmic(k, T, P, N, chunk, window, s_io, kept)
        rows.append((k, ms, by / (ms * 1e-3) / 1e9 if ms > 0 else 0.0, fl / (ms * 1e-3) / 1e12 if ms > 0 else 0.0,
                     ops / (ms * 1e-3) / 1e9 if ms > 0 else 0.0))
    if args.phases:
        print(f"{'phase':12s} {'ms':>9s} {'GB/s':>9s} {'TFLOP/s':>9s} {'VALU Gop/s':>11s}", file=sys.stderr)
        for k, ms, gbs, tfs, gops in rows:
            print(f"{k:12s} {ms:9.3f} {gbs:9.1f} {tfs:9.1f} {gops:11.1f}", file=sys.stderr)
        print(f"step {ms_per_step:.3f} ms (events), host wall {wall_ms / args.steps:.3f} ms/step", file=sys.stderr)

    # the dominant kernel
    dom = max(rows, key=lambda r: r[1])
    name, ms = dom[0], dom[1]
    by, fl, ops = algorithmic(name, T, P, N, chunk, window, s_io, kept)
    # per launch: the fused reverse kernel runs once per slab of chunks (equal
    # slabs at this workload), every other phase once per step
    nl = nslab if name == "bwd_main" else 1
    ms_l, by_l, fl_l, ops_l = ms / nl, by / nl, fl / nl, ops / nl
    hbm_ach = by_l / (ms_l * 1e-3) / 1e9
    if fl > 0:
        peak = MFMA_BF16_PEAK_TFS if io == "bf16" else MFMA_F32_PEAK_TFS
        ach = fl_l / (ms_l * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak}
    else:
        ach = ops_l / (ms_l * 1e-3) / 1e9
        roof = {"bound": "alu", "achieved": ach, "peak": VALU_PEAK_GOPS, "unit": "Gop/s",
                "frac": ach / VALU_PEAK_GOPS, "valu_frac": ach / VALU_PEAK_GOPS}
    # HBM bytes per launch from the stored counter reading (None if the kernel changed since)
    st = stored_traffic(name, args.workload)
    roof["traffic"] = None if st is None else st
    roof["traffic_unit"] = "bytes/launch"
    roof.update(kernel=name, launches_per_step=nl, ms=ms_l, algorithmic_bytes=by_l, hbm_achieved_gbs=hbm_ach,
                hbm_frac=hbm_ach / HBM_PEAK_GBS)

    out = {
        "metric": "SSM adjoint-gradient tokens/s (fwd+adjoint+VJP) at T=1M; % HBM roofline",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{case.name}: one selective SSM layer, T={T}, P={P}, N={N}, io={io}, "
                               f"fp32 state, window={window}, "
                               + {None: f"h stored only at {chunk}-token chunk boundaries (the gradient rebuilds "
                                        "the states inside each chunk)",
                                  "sub": f"h stored at {chunk}-token chunk boundaries and before every 8th token "
                                         "(the forward keeps the sub-chunk states)",
                                  "all": "every h_t stored by the forward and read by the gradient "
                                         "(the store-everything backpropagation baseline)"}[kept],
                   "T": T, "P": P, "N": N, "window": window, "chunk": chunk,
                   "states_kept": kept or "chunk checkpoints", "fused_kernel_launches": nslab,
                   "device_memory_gib": {
                       "saved_state": round(sum(v.numel() * v.element_size() for v in saved.values()) / 2**30, 3),
                       "gradient_workspace": round(ws_b.numel() / 2**30, 3),
                       "forward_workspace": round(ws_f.numel() / 2**30, 3),
                       "total_with_inputs_and_outputs": round(mem_total / 2**30, 3)}},
        "roofline": roof,
        "phases_ms": {k: round(v, 4) for k, v in phase_ms.items()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, window, chunk, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
