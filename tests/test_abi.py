"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, sizes its buffers, and rejects bad arguments before any
HIP call is made."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def agm():
    lib = os.path.join(ROOT, "adjoint_gradients_amd", "libssm_adjoint.so")
    if not os.path.exists(lib):
        pytest.fail("libssm_adjoint.so not built (run __graft_entry__.build())")
    import adjoint_gradients_amd as agm

    return agm


def test_header_functions_are_exported(agm):
    names = _declared_functions()
    assert set(names) == set(agm.EXPORTED), names
    for n in names:
        assert hasattr(agm.lib, n), n


def test_version_and_status_strings(agm):
    assert agm.ssm_version() >= 100
    for code, name in agm.STATUS.items():
        assert agm.ssm_status_str(code).startswith(name)
    assert agm.ssm_status_str(99) == "SSM_ERR_UNKNOWN"


def test_sizes(agm):
    d = agm.make_dims(1000, 48, 16, 64, "bf16")
    K = (1000 + 63) // 64
    saved = agm.ssm_saved_bytes(d)
    # s [T][P] f32, b and c [T][N] f32, h_ckpt [K][P][N] f32, s_sum [K][P] f64 (each 256-byte aligned)
    raw = 1000 * 48 * 4 + 2 * 1000 * 16 * 4 + K * 48 * 16 * 4 + K * 48 * 8
    assert raw <= saved <= raw + 5 * 256
    fwd = agm.ssm_workspace_bytes(d, 0, 0)
    bwd = agm.ssm_workspace_bytes(d, 100, 0)
    stk = agm.ssm_workspace_bytes(d, 100, 3)
    assert 0 < fwd < bwd < stk
    assert stk > 3 * saved


@pytest.mark.parametrize("T,P,N,C,io", [
    (0, 8, 4, 16, 0), (8, 0, 4, 16, 0), (8, 8, 0, 16, 0), (8, 8, 4, 0, 0),
])
def test_sizes_reject_bad_dims(agm, T, P, N, C, io):
    d = agm.Dims(T, P, N, C, io)
    assert agm.ssm_saved_bytes(d) == 0
    assert agm.ssm_workspace_bytes(d, 0, 0) == 0


@pytest.mark.parametrize("N,C,io", [(3, 16, 0), (128, 16, 0), (16, 513, 0), (16, 16, 2)])
def test_sizes_reject_unsupported(agm, N, C, io):
    d = agm.Dims(64, 8, N, C, io)
    assert agm.ssm_workspace_bytes(d, 0, 0) == 0


def _fake(addr=0x100000):
    """A non-null, 256-aligned fake device address (never dereferenced: every
    call below fails validation before any launch)."""
    return ctypes.c_void_p(addr)


def _layer(agm, misalign=False):
    a = 0x200000 + (4 if misalign else 0)
    return agm.Layer(a, 0x300000, 0x400000, 0x500000, None, None)


def _saved(agm, null_field=None):
    vals = dict(s=0x600000, b=0x700000, c=0x800000, h_ckpt=0x900000, s_sum=0xA00000)
    if null_field:
        vals[null_field] = None
    return agm.Saved(**vals)


def _grads(agm, null_field=None):
    vals = dict(dW_delta=0xB00000, dW_B=0xC00000, dW_C=0xD00000, dalpha=None, dbias=None, dx=None)
    if null_field:
        vals[null_field] = None
    return agm.Grads(**vals)


def _fwd(agm, d, layer, x, y, saved, ws, nbytes):
    return agm.lib.ssm_forward(ctypes.byref(d), ctypes.byref(layer) if layer is not None else None, x, y,
                               ctypes.byref(saved) if saved is not None else None, ws, nbytes, None)


def test_forward_validation(agm):
    d = agm.make_dims(64, 8, 4, 16)
    need = agm.ssm_workspace_bytes(d, 0, 0)
    L, S = _layer(agm), _saved(agm)
    x, y, ws = 0x1000000, 0x2000000, 0x3000000
    assert _fwd(agm, agm.Dims(0, 8, 4, 16, 0), L, x, y, S, ws, need) == 1
    assert _fwd(agm, agm.Dims(64, 8, 5, 16, 0), L, x, y, S, ws, need) == 4
    assert _fwd(agm, d, None, x, y, S, ws, need) == 1
    assert _fwd(agm, d, _layer(agm, misalign=True), x, y, S, ws, need) == 1
    assert _fwd(agm, d, L, None, y, S, ws, need) == 1
    assert _fwd(agm, d, L, x, None, S, ws, need) == 1
    assert _fwd(agm, d, L, x + 2, y, S, ws, need) == 1
    for f in ("s", "b", "c", "h_ckpt", "s_sum"):
        assert _fwd(agm, d, L, x, y, _saved(agm, f), ws, need) == 1, f
    assert _fwd(agm, d, L, x, y, S, None, need) == 2
    assert _fwd(agm, d, L, x, y, S, ws, need - 1) == 2
    assert _fwd(agm, d, L, x, y, S, ws + 16, need) == 2


def test_adjoint_validation(agm):
    d = agm.make_dims(64, 8, 4, 16)
    L, S = _layer(agm), _saved(agm)
    x, g, ws = 0x1000000, 0x2000000, 0x3000000
    need = agm.ssm_workspace_bytes(d, 8, 0)

    def call(window=8, grads=None, nbytes=need, wsp=ws, gp=g):
        G = grads if grads is not None else _grads(agm)
        return agm.lib.ssm_adjoint_grad(ctypes.byref(d), ctypes.byref(L), x, ctypes.byref(S), gp, window,
                                        ctypes.byref(G), wsp, nbytes, None)

    assert call(window=0) == 1
    assert call(window=-5) == 1
    assert call(gp=None) == 1
    for f in ("dW_delta", "dW_B", "dW_C"):
        assert call(grads=_grads(agm, f)) == 1, f
    assert call(nbytes=256) == 2
    assert call(wsp=None) == 2


def test_stack_validation(agm):
    d = agm.make_dims(64, 8, 4, 16)
    K = 2
    layers = (agm.Layer * K)(_layer(agm), _layer(agm))
    grads = (agm.Grads * K)(_grads(agm), _grads(agm))
    need = agm.ssm_workspace_bytes(d, 8, K)
    x0, g, ws = 0x1000000, 0x2000000, 0x3000000

    def call(K=K, window=8, ls=layers, gs=grads, nbytes=need):
        return agm.lib.ssm_stack_grad(K, ctypes.byref(d), ls, x0, g, window, gs, None, None, ws, nbytes, None)

    assert call(K=0) == 1
    assert call(window=0) == 1
    bad = (agm.Layer * K)(_layer(agm), _layer(agm, misalign=True))
    assert call(ls=bad) == 1
    with_dx = (agm.Grads * K)(_grads(agm), agm.Grads(0xB00000, 0xC00000, 0xD00000, None, None, 0xE00000))
    assert call(gs=with_dx) == 1
    assert call(nbytes=256) == 2


def test_gradient_workspace_is_bounded(agm):
    # the 1M-token layer (T = 2^20, P = 2048, N = 16, bf16, chunk 256, window
    # 4096): without sub-chunk states kept by the forward, the gradient
    # rebuilds them slab by slab in a region of at most 1 GiB; dx_dir lives
    # in the dx output, so the workspace is the GEMM operand, the channel
    # partials, the chunk aggregates and that region
    gib = 1 << 30
    d = agm.make_dims(1 << 20, 2048, 16, 256, "bf16")
    full = agm.ssm_workspace_bytes(d, 4096, 0)
    sub = agm.ssm_grad_workspace_bytes_sub(d, 4096)
    assert full <= 10 * gib, full / gib
    assert 0 < full - sub <= gib
    assert agm.ssm_sub_state_bytes(d) == (1 << 20) // 8 * 2048 * 16 * 4
    slabs = agm.ssm_grad_slab_count(d, 4096, False)
    assert slabs == 16 and agm.ssm_grad_slab_count(d, 4096, True) == 1
    # doubling T doubles the slab count, not the region
    d2 = agm.make_dims(1 << 21, 2048, 16, 256, "bf16")
    assert agm.ssm_grad_slab_count(d2, 4096, False) == 2 * slabs
    assert agm.ssm_workspace_bytes(d2, 4096, 0) - agm.ssm_grad_workspace_bytes_sub(d2, 4096) == full - sub
    # a short sequence: one slab holding every chunk
    d3 = agm.make_dims(1000, 48, 16, 64, "f32")
    assert agm.ssm_grad_slab_count(d3, 100, False) == 1


def test_slabs_start_at_carry_segment_multiples(agm):
    # A slab holds at most 1 GiB of sub-chunk states (C / 8 state vectors of
    # P N floats per chunk), rounded down to a multiple of 32 chunks when that
    # many fit, else of 16 (the carry between chunks is scanned in segments of
    # 16 at fixed positions, so slab starts at multiples of 16 keep every
    # carry independent of the slab size).
    def slabs(T, P, N):
        return agm.ssm_grad_slab_count(agm.make_dims(T, P, N, 256, "bf16"), 4096, False)

    per = lambda P, N: 32 * P * N * 4  # bytes of one chunk's sub-chunk states
    # 1 GiB holds 21 chunks at P = 6144, N = 64: rounded down to 16
    assert (1 << 30) // per(6144, 64) == 21
    assert slabs(256 * 100, 6144, 64) == 7  # ceil(100 / 16)
    # 1 GiB holds 39 chunks at P = 3328, N = 64: rounded down to 32
    assert (1 << 30) // per(3328, 64) == 39
    assert slabs(256 * 100, 3328, 64) == 4  # ceil(100 / 32)
    # fewer than 16 fit: no rounding (12 chunks at P = 10240, N = 64)
    assert (1 << 30) // per(10240, 64) == 12
    assert slabs(256 * 100, 10240, 64) == 9  # ceil(100 / 12)


def test_stack_workspace_counts_normalising_layers(agm):
    d = agm.make_dims(1000, 48, 16, 64, "f32")
    plain = (agm.Layer * 3)(_layer(agm), _layer(agm), _layer(agm))
    one = (agm.Layer * 3)(_layer(agm), agm.Layer(0x200000, 0x300000, 0x400000, 0x500000, None, 0xF00000),
                          _layer(agm))
    base = agm.lib.ssm_stack_workspace_bytes(3, ctypes.byref(d), plain, 100)
    assert base == agm.ssm_workspace_bytes(d, 100, 3) > 0
    with_norm = agm.lib.ssm_stack_workspace_bytes(3, ctypes.byref(d), one, 100)
    # one layer's r^k (T P floats) and 1/rms (T floats), one dx (T P), row scratch
    assert with_norm - base >= (2 * 1000 * 48 + 2 * 1000) * 4
    # a stack with a normalising layer and only the plain size is refused
    grads = (agm.Grads * 3)(_grads(agm), _grads(agm), _grads(agm))
    rc = agm.lib.ssm_stack_grad(3, ctypes.byref(d), one, 0x1000000, 0x2000000, 100, grads, None, None,
                                0x3000000, base, None)
    assert rc == 2


def test_binding_checks_tensors_before_the_call(agm):
    import torch

    d = agm.make_dims(64, 8, 4, 16)
    x = torch.zeros(64, 8)
    with pytest.raises(agm.SsmError, match="GPU tensor"):
        agm._need(x, "x", 64 * 8, torch.float32)
    if torch.cuda.is_available():
        x = x.cuda()
        with pytest.raises(agm.SsmError, match="contiguous"):
            agm._need(x.t(), "x", 64 * 8, torch.float32)
        with pytest.raises(agm.SsmError, match="dtype"):
            agm._need(x.to(torch.bfloat16), "x", 64 * 8, torch.float32)
        with pytest.raises(agm.SsmError, match="elements"):
            agm._need(x[:32], "x", 64 * 8, torch.float32)
    with pytest.raises(agm.SsmError, match="required"):
        agm.saved_struct({}, d)


def test_noalloc_refuses_oversize_before_launch(agm):
    # the 1M-token layer's fixed gradient buffers (GB) exceed the library's
    # array: refused by the size check, before any device call
    d = agm.make_dims(1 << 20, 2048, 16, 256, "bf16")
    L, S, G = _layer(agm), _saved(agm), _grads(agm)
    rc = agm.lib.ssm_adjoint_grad_noalloc(ctypes.byref(d), ctypes.byref(L), 0x1000000, ctypes.byref(S),
                                          0x2000000, 4096, ctypes.byref(G), None)
    assert rc == 2
    # argument errors come first, as in ssm_adjoint_grad
    rc = agm.lib.ssm_adjoint_grad_noalloc(ctypes.byref(d), ctypes.byref(L), 0x1000000, ctypes.byref(S),
                                          0x2000000, 0, ctypes.byref(G), None)
    assert rc == 1


def test_probe_validation(agm):
    # the unit probes reject bad arguments before any HIP call (fake
    # non-null addresses are never dereferenced)
    L = agm.lib
    sink, clk = ctypes.c_void_p(0x600000), ctypes.c_void_p(0x700000)
    for kind, wgs, iters, s, c in [(-1, 8, 10, sink, clk), (4, 8, 10, sink, clk), (0, 0, 10, sink, clk),
                                   (0, (1 << 20) + 1, 10, sink, clk), (0, 8, 0, sink, clk),
                                   (0, 8, 1 << 31, sink, clk), (3, 8, 10, None, clk), (3, 8, 10, sink, None)]:
        assert L.ssm_probe_units(kind, wgs, iters, s, c, None) == 1, (kind, wgs, iters)
    assert L.ssm_probe_wall_clock_khz(None) == 1
