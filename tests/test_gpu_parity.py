"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerance: per-tensor max|gpu - ref| / max|ref| <= 1e-4 for fp32 inputs and
<= 2e-2 for bf16 inputs with fp32 state.  Every case prints its label before
running so a failure names it.
"""
import numpy as np
import pytest

from gpu_util import GRAD_KEYS, TOL, compare, gpu_layer, oracle_inputs, rel_err, say
from ssm_inputs import CASES, LayerCase, make_layer, make_stack, small_case, window_pin_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import adjoint_gradients_amd  # noqa: F401  (fails loudly if the library is missing)


@pytest.fixture(scope="module")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


def _run_case(orc, inp, window, chunk, label, tol=None, sub_states=False, all_states=False):
    say(f"case {label}: T={inp['x'].shape[0]} P={inp['x'].shape[1]} N={inp['W_B'].shape[0]} "
        f"io={inp['io']} W={window} C={chunk} sub_states={sub_states} all_states={all_states}")
    tol = tol if tol is not None else TOL[inp["io"]]
    got = gpu_layer(inp, window, chunk, sub_states=sub_states, all_states=all_states)
    o = oracle_inputs(inp)
    T = inp["x"].shape[0]
    ref = orc.layer_grad(o, window=None if window >= T else window)
    compare(got, ref, GRAD_KEYS, tol, label)
    # saved state: s = softplus(Delta), b, c, checkpoints
    s_ref = np.logaddexp(0.0, ref["delta"])
    assert rel_err(got["saved_s"], s_ref) <= tol
    assert rel_err(got["saved_b"], ref["b"]) <= tol
    assert rel_err(got["saved_c"], ref["c"]) <= tol
    hck = orc.forward(o, C=chunk)["h_ckpt"]
    assert rel_err(got["saved_h_ckpt"], hck) <= tol
    return got, ref


def test_layer256_exact(orc):
    inp = make_layer(CASES[0])
    _run_case(orc, inp, 256, 256, "256-token layer W=T")


@pytest.mark.parametrize("chunk", [1, 3, 16, 100, 256, 512])
def test_chunk_invariance_ragged(orc, chunk):
    inp = make_layer(small_case(300, 40, 8, 5))
    _run_case(orc, inp, 300, chunk, f"ragged C={chunk}")


@pytest.mark.parametrize("N,chunk", [(64, 256), (32, 512), (64, 100)])
def test_rebuild_rows_in_parts(orc, N, chunk):
    """Chunks whose b and c rows exceed the staging areas are staged in parts
    (the rebuild: 128 tokens at N = 64, 256 at N = 32; the forward: 64 or 128
    tokens at N = 64, 128 or 256 at N = 32): chunk checkpoints only, a window
    of whole chunks and exact, with a ragged last chunk and channel blocks
    that do not fill the last workgroup.  C = 100 at N = 64 stages the
    forward in a part of 64 tokens and one of 36 (chunks that are not whole
    ring turns)."""
    inp = make_layer(small_case(1100 if chunk == 512 else 700, 40, N, 30 + N))
    T = inp["x"].shape[0]
    _run_case(orc, inp, chunk, chunk, f"rows in parts N={N} C={chunk} W={chunk}")
    _run_case(orc, inp, T, chunk, f"rows in parts N={N} C={chunk} exact")


@pytest.mark.parametrize("N", [1, 2, 4, 16, 32, 64])
def test_state_sizes(orc, N):
    inp = make_layer(small_case(200, 70, N, 6 + N))
    _run_case(orc, inp, 200, 32, f"N={N}")
    _run_case(orc, inp, 37, 32, f"N={N} W=37")


@pytest.mark.parametrize("W", [1, 2, 3, 7, 64, 255, 256, 511, 512, 513])
def test_window_pinning(orc, W):
    """Slow decay: adjacent windows differ by far more than the tolerance."""
    inp = make_layer(window_pin_case(seed=100, T=512, P=8, N=4))
    got, ref = _run_case(orc, inp, W, 64, f"winpin W={W}")
    if W < 512:
        exact = orc.layer_grad(oracle_inputs(inp), window=None)
        gap = rel_err(ref["dx"], exact["dx"])
        err = rel_err(got["dx"], ref["dx"])
        say(f"  window-vs-exact gap (dx) = {gap:.2e}")
        # a kernel that ran another window (W - 1, W + 1, or none) would miss
        # the oracle by about this gap: it must be far above the error
        assert err < gap / 100, (W, err, gap)


@pytest.mark.parametrize("chunk", [7, 64, 200])
def test_window_chunk_not_dividing(orc, chunk):
    inp = make_layer(window_pin_case(seed=101, T=700, P=8, N=4))
    for W in (5, 130, 333):
        _run_case(orc, inp, W, chunk, f"winpin C={chunk} W={W}")


@pytest.mark.parametrize("chunk,W", [(32, 32), (32, 96), (64, 320), (100, 300), (128, 640)])
def test_window_whole_chunks(orc, chunk, W):
    """Windows of whole chunks: the window terms of a chunk's aggregate come
    from the exact aggregate W tokens later.  T = 700 leaves a ragged last
    chunk, and the slow decay keeps every dropped term visible."""
    inp = make_layer(window_pin_case(seed=102, T=700, P=8, N=4))
    got, ref = _run_case(orc, inp, W, chunk, f"winpin whole chunks C={chunk} W={W}")
    exact = orc.layer_grad(oracle_inputs(inp), window=None)
    gap = rel_err(ref["dx"], exact["dx"])
    say(f"  window-vs-exact gap (dx) = {gap:.2e}")
    assert rel_err(got["dx"], ref["dx"]) < gap / 100, (chunk, W, gap)


def test_window_whole_chunks_bf16_n16(orc):
    inp = make_layer(small_case(1000, 96, 16, 21, io="bf16"))
    for W in (128, 384):
        _run_case(orc, inp, W, 128, f"bf16 N=16 whole-chunk window W={W}")


def test_bf16_small(orc):
    c = small_case(1024, 96, 16, 9, io="bf16")
    inp = make_layer(c)
    _run_case(orc, inp, 1024, 256, "bf16 W=T")
    _run_case(orc, inp, 200, 256, "bf16 W=200")


@pytest.mark.parametrize("T,P", [(64, 32), (96, 64), (160, 96), (128, 160), (32, 128)])
def test_bf16_short_k(orc, T, P):
    # bf16 GEMMs with 1 to 5 k-steps of 32 (projection K = P, weight gradient
    # K = T split over blocks): pipeline fill and drain with fewer steps than
    # LDS stages
    c = small_case(T, P, 16, 11, io="bf16")
    inp = make_layer(c)
    _run_case(orc, inp, T, 32, f"bf16 short-k T={T} P={P}")


@pytest.mark.parametrize("label,T,P,N,io,window,chunk", [
    ("exact", 256, 64, 16, "f32", 256, 256),
    ("ragged C", 300, 40, 8, "f32", 300, 100),
    ("C < sub-chunk", 300, 40, 8, "f32", 300, 3),
    ("window", 1024, 96, 16, "f32", 255, 256),
    ("window C not dividing", 700, 70, 16, "f32", 200, 7),
    ("N=1", 300, 40, 1, "f32", 120, 64),
    ("N=64", 512, 48, 64, "f32", 200, 256),
    ("bf16", 1024, 96, 16, "bf16", 200, 256),
])
def test_sub_states(orc, label, T, P, N, io, window, chunk):
    # the forward keeps the sub-chunk states and the gradient skips its own
    # pass: same oracle tolerance, and the same result as without them
    inp = make_layer(small_case(T, P, N, 21, io=io))
    got, _ = _run_case(orc, inp, window, chunk, f"sub-states {label}", sub_states=True)
    ref = gpu_layer(inp, window, chunk, sub_states=False)
    for gk, _ in GRAD_KEYS:
        assert rel_err(got[gk], ref[gk]) <= 1e-5, gk


@pytest.mark.parametrize("label,T,P,N,io,window,chunk", [
    ("exact", 256, 64, 16, "f32", 256, 256),
    ("ragged C", 300, 40, 8, "f32", 300, 100),
    ("window", 1024, 96, 16, "f32", 255, 256),
    ("window of whole chunks, ragged T", 700, 70, 32, "f32", 256, 128),
    ("N=1", 300, 40, 1, "f32", 120, 64),
    ("N=64, one-wavefront forward", 512, 48, 64, "f32", 200, 256),
    ("bf16", 1024, 96, 16, "bf16", 200, 256),
])
def test_store_everything_baseline(orc, label, T, P, N, io, window, chunk):
    # the forward keeps every state (h_all) and the gradient reads them
    # instead of rebuilding any: the oracle's tolerance, and the same result
    # as the path that keeps only the chunk checkpoints
    inp = make_layer(small_case(T, P, N, 22, io=io))
    got, _ = _run_case(orc, inp, window, chunk, f"store-everything {label}", all_states=True)
    ref = gpu_layer(inp, window, chunk)
    for gk, _ in GRAD_KEYS:
        assert rel_err(got[gk], ref[gk]) <= 1e-6, gk


@pytest.mark.parametrize("mode", ["checkpoints", "sub_states", "all_states"])
@pytest.mark.parametrize("T,P,N,io,window,chunk", [
    (512, 48, 64, "f32", 200, 256),    # 6 channel blocks: idle wavefronts in the last workgroup
    (300, 40, 8, "f32", 120, 100),
    (1024, 96, 16, "bf16", 200, 256),
    (700, 70, 32, "f32", 700, 64),
    (1000, 96, 16, "bf16", 256, 128),  # window of whole chunks, ragged last chunk, an idle wavefront
    (700, 40, 8, "f32", 200, 100),     # window of whole chunks, one lane group
])
def test_poisoned_buffers(orc, T, P, N, io, window, chunk, mode):
    # workspaces and saved buffers filled with NaN bytes beforehand: a read of
    # anything the library did not write shows up in the outputs
    import torch

    import adjoint_gradients_amd as agm
    from gpu_util import layer_tensors, to_dev

    inp = make_layer(small_case(T, P, N, 31, io=io))
    sub_states, all_states = mode == "sub_states", mode == "all_states"
    say(f"case poisoned T={T} P={P} N={N} io={io} W={window} C={chunk} kept={mode}")
    dims = agm.make_dims(T, P, N, chunk, io)
    lay = layer_tensors(inp, io)
    x = to_dev(inp["x"], io)
    g = to_dev(inp["g"])
    ws_f = agm.alloc_workspace(agm.ssm_workspace_bytes(dims, 0, 0), x.device).fill_(255)
    nb = (agm.ssm_grad_workspace_bytes_sub(dims, window) if mode != "checkpoints"
          else agm.ssm_workspace_bytes(dims, window, 0))
    ws_b = agm.alloc_workspace(nb, x.device).fill_(255)
    saved = agm.alloc_saved(dims, x.device, sub_states=sub_states, all_states=all_states)
    for v in saved.values():
        v.view(torch.uint8).fill_(255)
    y, saved = agm.forward(dims, lay, x, ws=ws_f, saved=saved)
    grads = agm.adjoint_grad(dims, lay, x, saved, g, window, want_dx=True, ws=ws_b)
    torch.cuda.synchronize()
    got = {k: v.double().cpu().numpy() for k, v in grads.items()}
    got["y"] = y.double().cpu().numpy()
    ref = orc.layer_grad(oracle_inputs(inp), window=None if window >= T else window)
    compare(got, ref, GRAD_KEYS, TOL[io], f"poisoned N={N} P={P} kept={mode}")


@pytest.mark.parametrize("io,window,mask", [("f32", 256, (1, 1, 1)), ("f32", 50, (1, 0, 1)),
                                            ("bf16", 256, (1, 1, 1)), ("bf16", 50, (0, 1, 1)),
                                            ("f32", 50, (1, 1, 0))])
def test_stack_normalised(orc, io, window, mask):
    # layers reading the RMS-normalised residual stream (mask: which layers
    # normalise); every gradient, dgamma, dx0 and r^K against the oracle
    c = LayerCase("stack_norm", 256, 48, 16, io, (), K=3, seed=41)
    st = make_stack(c)
    rng = np.random.default_rng(42)
    for lay, m in zip(st["layers"], mask):
        if m:
            lay["norm_scale"] = rng.uniform(0.5, 1.5, 48).astype(np.float32)
    say(f"case normalised stack K=3 io={io} W={window} mask={mask}")
    grads, dx0, xK = _gpu_stack(st, window, 64)
    st64 = dict(st, x=np.asarray(st["x"], np.float64), g=np.asarray(st["g"], np.float64),
                layers=[{k: np.asarray(v, np.float64) for k, v in lay.items()} for lay in st["layers"]])
    ref = orc.stack_grad(st64, window=None if window >= 256 else window)
    tol = TOL[io]
    for k in range(3):
        names = ["dW_delta", "dW_B", "dW_C", "dalpha", "dbias"] + (["dnorm_scale"] if mask[k] else [])
        compare(grads[k], ref["layers"][k], [(n, n) for n in names], tol, f"normalised stack layer {k}")
    assert rel_err(dx0, ref["dx0"]) <= tol
    assert rel_err(xK, ref["forward"]["r_final"]) <= tol


def test_single_layer_rejects_norm_scale():
    import adjoint_gradients_amd as agm
    from gpu_util import layer_tensors, to_dev

    inp = make_layer(small_case(64, 16, 4, 43))
    inp["norm_scale"] = np.ones(16, dtype=np.float32)
    dims = agm.make_dims(64, 16, 4, 64, "f32")
    with pytest.raises(agm.SsmError):
        agm.forward(dims, layer_tensors(inp, "f32"), to_dev(inp["x"]))


def test_determinism_and_linearity():
    import adjoint_gradients_amd as agm  # noqa: F401

    inp = make_layer(small_case(500, 80, 16, 12))
    a = gpu_layer(inp, 120, 64)
    b = gpu_layer(inp, 120, 64)
    for k in ("dW_delta", "dW_B", "dW_C", "dalpha", "dbias", "dx", "y"):
        assert np.array_equal(a[k], b[k]), k
    c = gpu_layer(inp, 120, 64, g=2.0 * inp["g"])
    for k in ("dW_delta", "dW_B", "dW_C", "dalpha", "dbias", "dx"):
        assert np.array_equal(c[k], 2.0 * a[k]), k


def test_slabs_ragged(orc):
    # 300 chunks of 256 tokens at P = 1024, N = 32 (4 MiB of sub-chunk states
    # per chunk): the gradient rebuilds them in slabs of 256 chunks (1 GiB),
    # so the second slab is a ragged one of 44.  fp32, a window (1000) that is
    # not a whole number of chunks and the exact gradient, with the states
    # rebuilt slab by slab and with them kept by the forward.
    T, P, N, C = 300 * 256, 1024, 32, 256
    inp = make_layer(small_case(T, P, N, 51))
    o = oracle_inputs(inp)
    for W in (1000, T):
        ref = orc.layer_grad(o, window=None if W >= T else W)
        for sub in (False, True):
            label = f"slabs T={T} P={P} N={N} W={W} sub_states={sub}"
            say(f"case {label}")
            got = gpu_layer(inp, W, C, sub_states=sub)
            compare(got, ref, GRAD_KEYS, TOL["f32"], label)


def test_layer16k(orc):
    inp = make_layer(CASES[1])
    for W in (16384, 2048):
        _run_case(orc, inp, W, 256, f"16K-token layer W={W}")


def _gpu_stack(st, window, chunk):
    import torch

    import adjoint_gradients_amd as agm
    from gpu_util import layer_tensors, to_dev

    io = st["io"]
    T, P = st["x"].shape
    N = st["layers"][0]["W_B"].shape[0]
    dims = agm.make_dims(T, P, N, chunk, io)
    lays = [layer_tensors(lay, io) for lay in st["layers"]]
    grads, dx0, xK = agm.stack_grad(dims, lays, to_dev(st["x"], io), to_dev(st["g"]), window)
    torch.cuda.synchronize()
    return ([{k: v.double().cpu().numpy() for k, v in g.items()} for g in grads],
            dx0.double().cpu().numpy(), xK.double().cpu().numpy())


@pytest.mark.parametrize("io,window", [("f32", 256), ("f32", 50), ("bf16", 256), ("bf16", 50)])
def test_stack(orc, io, window):
    c = LayerCase("stack_small", 256, 48, 16, io, (), K=3, seed=40)
    st = make_stack(c)
    say(f"case stack K=3 io={io} W={window}")
    grads, dx0, xK = _gpu_stack(st, window, 64)
    st64 = dict(st, x=np.asarray(st["x"], np.float64), g=np.asarray(st["g"], np.float64),
                layers=[{k: np.asarray(v, np.float64) for k, v in lay.items()} for lay in st["layers"]])
    ref = orc.stack_grad(st64, window=None if window >= 256 else window)
    tol = TOL[io]
    for k in range(3):
        compare(grads[k], ref["layers"][k], [(n, n) for n in ("dW_delta", "dW_B", "dW_C", "dalpha", "dbias")],
                tol, f"stack layer {k}")
    assert rel_err(dx0, ref["dx0"]) <= tol
    assert rel_err(xK, ref["forward"]["r_final"]) <= tol
