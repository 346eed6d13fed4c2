"""Pins of the fp64 oracle against things other than itself.

Each test checks one oracle function against a result that the pages or the
mathematics fix independently: library routines (numpy matmul / cumsum, torch
float64 autograd, torch bfloat16 casts), closed forms, finite differences of
the oracle's *forward* only, and brute force on tiny inputs.  Citations refer
to the review of "Adjoint sharding for very long context training of state
space models" (arXiv 2501.00692).
"""
import math

import numpy as np
import pytest

from conftest import rel_err
from ssm_inputs import LayerCase, make_layer, make_stack, small_case, window_pin_case


def _tiny(T=24, P=4, N=3, seed=7, bias="zero"):
    c = small_case(T, P, N, seed, bias=bias)
    d = make_layer(c)
    return {k: (np.asarray(v, dtype=np.float64) if isinstance(v, np.ndarray) else v) for k, v in d.items()}


# ---------------------------------------------------------------- projections

def test_projection_matches_library_matmul(orc):
    inp = _tiny(T=37, P=9, N=5)
    pr = orc.projections(inp)
    ref_d = inp["x"] @ inp["W_delta"].T + inp["delta_bias"]
    assert rel_err(pr["delta"], ref_d) < 1e-14
    assert rel_err(pr["b"], inp["x"] @ inp["W_B"].T) < 1e-14
    assert rel_err(pr["c"], inp["x"] @ inp["W_C"].T) < 1e-14


def test_blas_projection_and_channel_sums_match_loops(orc):
    # the matmul path used for the million-token workloads equals the loops
    inp = _tiny(T=300, P=24, N=4)
    chans = np.array([0, 5, 23])
    a = orc.channel_grad(inp, chans, window=37)
    b = orc.channel_grad(inp, chans, window=37, blas=True)
    pr = orc.projections(inp, blas=True)
    c = orc.channel_grad(inp, chans, window=37, blas=True, bc={"b": pr["b"], "c": pr["c"]})
    for k in ("y", "dDelta", "dalpha", "dbias", "db_part", "dc_part", "dW_delta_rows"):
        assert rel_err(b[k], a[k]) < 1e-12, k
        assert rel_err(c[k], a[k]) < 1e-12, k
    assert rel_err(orc.project(inp["x"], inp["W_delta"], inp["delta_bias"], block=64, blas=True),
                   orc.project(inp["x"], inp["W_delta"], inp["delta_bias"])) < 1e-14


def test_time_sums_match_library_matmul(orc):
    rng = np.random.default_rng(3)
    T, P, M = 53, 7, 6
    dY = rng.standard_normal((T, M))
    x = rng.standard_normal((T, P))
    W = rng.standard_normal((M, P))
    lib = orc._load()
    dW = np.empty((M, P))
    lib.orc_weight_grad(T, P, M, orc._pd(dY), orc._pd(x), orc._pd(dW))
    assert rel_err(dW, dY.T @ x) < 1e-14
    dx = np.zeros((T, P))
    lib.orc_input_grad(T, P, M, orc._pd(dY), orc._pd(W), orc._pd(dx))
    assert rel_err(dx, dY @ W) < 1e-14


# ---------------------------------------------------------------- forward

def test_forward_alpha_zero_is_cumulative_sum(orc):
    """alpha = 0 => a = 1 => h_t = sum_{j<=t} b_j x_j (Section 3.1 recurrence)."""
    inp = _tiny(T=50, P=5, N=4)
    inp["alpha"] = np.zeros_like(inp["alpha"])
    out = orc.forward(inp)
    b, c, x = out["b"], out["c"], inp["x"]
    H = np.cumsum(x[:, :, None] * b[:, None, :], axis=0)
    y_ref = np.einsum("tpn,tn->tp", H, c)
    assert rel_err(out["y"], y_ref) < 1e-13


def test_forward_geometric_closed_form(orc):
    """P = N = 1, x = 1, W_delta = 0: constant a, h_t = b (1 - a^{t+1}) / (1 - a)."""
    T = 300
    beta, b0, c0, al = -1.3, 0.7, -1.9, 2.5
    inp = {"x": np.ones((T, 1)), "W_delta": np.zeros((1, 1)), "delta_bias": np.array([beta]),
           "W_B": np.array([[b0]]), "W_C": np.array([[c0]]), "alpha": np.array([[al]]),
           "g": np.ones((T, 1))}
    y = orc.forward(inp)["y"][:, 0]
    s = math.log1p(math.exp(beta))
    a = math.exp(-s * al)
    t = np.arange(T)
    y_ref = c0 * b0 * (1.0 - a ** (t + 1)) / (1.0 - a)
    assert rel_err(y, y_ref) < 1e-13


def test_forward_checkpoints_are_states(orc):
    """h_ckpt[k] = h_{kC-1}: the C = 1 run lists every state; any C subsamples it."""
    inp = _tiny(T=45, P=3, N=4)
    every = orc.forward(inp, C=1)["h_ckpt"]
    for C in (2, 7, 16, 45, 64):
        hc = orc.forward(inp, C=C)["h_ckpt"]
        assert hc.shape[0] == (45 + C - 1) // C
        assert np.array_equal(hc, every[::C])
    assert np.all(every[0] == 0.0)


# ---------------------------------------------------------------- exact gradient

def _fd_grad(f, arr, eps=2.0 ** -10):
    """Central differences with one Richardson step (error O(eps^4))."""
    g = np.empty_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        v = arr[idx]

        def d(e):
            arr[idx] = v + e
            fp = f()
            arr[idx] = v - e
            fm = f()
            arr[idx] = v
            return (fp - fm) / (2 * e)

        g[idx] = (4.0 * d(eps / 2) - d(eps)) / 3.0
    return g


@pytest.mark.parametrize("seed", [11, 12])
def test_exact_gradient_matches_finite_differences(orc, seed):
    """Window >= T: the summed VJPs equal the gradient of L = sum <g, y> (Proposition 2)."""
    inp = _tiny(T=20, P=4, N=3, seed=seed)
    gr = orc.layer_grad(inp, window=None)
    f = lambda: orc.loss(inp)
    checks = {
        "W_delta": "dW_delta", "W_B": "dW_B", "W_C": "dW_C",
        "alpha": "dalpha", "delta_bias": "dbias", "x": "dx",
    }
    for pname, gname in checks.items():
        fd = _fd_grad(f, inp[pname])
        assert rel_err(gr[gname], fd) < 1e-8, (pname, rel_err(gr[gname], fd))


def _torch_forward(th, T, N):
    """Plain float64 torch forward of the layer (used only for autograd pins)."""
    import torch

    x, Wd, bias, Wb, Wc, al = th["x"], th["W_delta"], th["delta_bias"], th["W_B"], th["W_C"], th["alpha"]
    delta = x @ Wd.T + bias
    b = x @ Wb.T
    c = x @ Wc.T
    s = torch.nn.functional.softplus(delta)
    h = torch.zeros(x.shape[1], N, dtype=torch.float64)
    ys = []
    for t in range(T):
        a = torch.exp(-s[t][:, None] * al)
        h = a * h + x[t][:, None] * b[t][None, :]
        ys.append(h @ c[t])
    return torch.stack(ys)


def test_exact_gradient_matches_torch_autograd(orc):
    torch = pytest.importorskip("torch")
    inp = _tiny(T=64, P=6, N=4, seed=21)
    gr = orc.layer_grad(inp, window=None)
    th = {k: torch.tensor(inp[k], requires_grad=True) for k in
          ("x", "W_delta", "delta_bias", "W_B", "W_C", "alpha")}
    y = _torch_forward(th, 64, 4)
    L = (torch.tensor(inp["g"]) * y).sum()
    L.backward()
    assert rel_err(gr["y"], y.detach().numpy()) < 1e-13
    for pname, gname in (("x", "dx"), ("W_delta", "dW_delta"), ("delta_bias", "dbias"),
                         ("W_B", "dW_B"), ("W_C", "dW_C"), ("alpha", "dalpha")):
        assert rel_err(gr[gname], th[pname].grad.numpy()) < 1e-12, pname


# ---------------------------------------------------------------- truncated (windowed) sums

def _per_token_truncated_autograd(inp, W):
    """Brute-force definition of truncated adjoint sharding ("Core claim").

    Every token i gets its own copy of the parameters (used only by token i's
    A_i, B_i, C_i).  The truncated gradient is sum_t sum_{t-W < i <= t} of
    d l_t / d theta_i, with h kept exact.  Computed by torch autograd, one
    backward pass per t.
    """
    import torch

    T, P = inp["x"].shape
    N = inp["W_B"].shape[0]
    names = ("W_delta", "delta_bias", "W_B", "W_C", "alpha")
    copies = {k: torch.tensor(np.repeat(inp[k][None], T, axis=0), requires_grad=True) for k in names}
    x = torch.tensor(inp["x"], requires_grad=True)
    g = torch.tensor(inp["g"])
    h = torch.zeros(P, N, dtype=torch.float64)
    ys = []
    for t in range(T):
        Wd, bi, Wb, Wc, al = (copies[k][t] for k in names)
        d = Wd @ x[t] + bi
        s = torch.nn.functional.softplus(d)
        a = torch.exp(-s[:, None] * al)
        h = a * h + x[t][:, None] * (Wb @ x[t])[None, :]
        ys.append(h @ (Wc @ x[t]))
    acc = {k: np.zeros_like(inp[k]) for k in names}
    acc_x = np.zeros_like(inp["x"])
    for t in range(T):
        lt = (g[t] * ys[t]).sum()
        grads = torch.autograd.grad(lt, [copies[k] for k in names] + [x], retain_graph=True)
        lo = max(0, t - W + 1)
        for k, gk in zip(names, grads[:-1]):
            acc[k] += gk[lo:t + 1].sum(0).numpy()
        acc_x[lo:t + 1] += grads[-1][lo:t + 1].numpy()
    return acc, acc_x


@pytest.mark.parametrize("W", [1, 2, 5, 16])
def test_truncated_matches_per_token_autograd(orc, W):
    pytest.importorskip("torch")
    inp = _tiny(T=16, P=3, N=3, seed=31)
    acc, acc_x = _per_token_truncated_autograd(inp, W)
    for method in ("literal", "identity"):
        gr = orc.layer_grad(inp, window=W, method=method)
        for pname, gname in (("W_delta", "dW_delta"), ("delta_bias", "dbias"), ("W_B", "dW_B"),
                             ("W_C", "dW_C"), ("alpha", "dalpha")):
            assert rel_err(gr[gname], acc[pname]) < 1e-11, (method, W, pname)
        assert rel_err(gr["dx"], acc_x) < 1e-11, (method, W, "x")


def test_window_one_closed_form(orc):
    """W = 1 keeps only lambda_{t,t} = C_t: mu_i = g_i c_i."""
    inp = _tiny(T=30, P=5, N=4, seed=41)
    gr = orc.layer_grad(inp, window=1)
    g, x, b, c = inp["g"], inp["x"], gr["b"], gr["c"]
    assert rel_err(gr["db"], c * np.sum(g * x, axis=1)[:, None]) < 1e-13
    assert rel_err(gr["dxdir"], g * np.sum(c * b, axis=1)[:, None]) < 1e-13


@pytest.mark.parametrize("W", [1, 3, 8, 29])
def test_alpha_zero_window_is_moving_sum(orc, W):
    """alpha = 0 => prod a = 1 => mu_i = sum_{t=i}^{i+W-1} g_t c_t (cumsum differences)."""
    inp = _tiny(T=30, P=4, N=3, seed=43)
    inp["alpha"] = np.zeros_like(inp["alpha"])
    gr = orc.layer_grad(inp, window=W)
    g, x, b, c = inp["g"], inp["x"], gr["b"], gr["c"]
    T = g.shape[0]
    gc = g[:, :, None] * c[:, None, :]
    cs = np.concatenate([np.zeros((1,) + gc.shape[1:]), np.cumsum(gc, axis=0)])
    hi = np.minimum(np.arange(T) + W, T)
    mu = cs[hi] - cs[np.arange(T)]
    assert rel_err(gr["db"], np.einsum("tpn,tp->tn", mu, x)) < 1e-12
    assert rel_err(gr["dxdir"], np.einsum("tpn,tn->tp", mu, b)) < 1e-12
    H = np.cumsum(x[:, :, None] * b[:, None, :], axis=0)
    Hprev = np.concatenate([np.zeros((1,) + H.shape[1:]), H[:-1]])
    s = np.log1p(np.exp(gr["delta"]))
    dal_ref = -np.einsum("tpn,tpn,tp->pn", mu, Hprev, s)
    assert rel_err(gr["dalpha"], dal_ref) < 1e-12
    assert np.max(np.abs(gr["dDelta"])) == 0.0


def test_literal_equals_bptt_and_identity(orc):
    inp = _tiny(T=40, P=5, N=3, seed=51, bias="zero")
    T = 40
    ref = orc.layer_grad(inp, window=T, method="bptt")
    lit = orc.layer_grad(inp, window=T, method="literal")
    for k in ("dW_delta", "dW_B", "dW_C", "dalpha", "dbias", "dx"):
        assert rel_err(lit[k], ref[k]) < 1e-12, k
    for W in (1, 2, 7, 16, T - 1):
        a = orc.layer_grad(inp, window=W, method="literal")
        b = orc.layer_grad(inp, window=W, method="identity")
        for k in ("dW_delta", "dW_B", "dW_C", "dalpha", "dbias", "dx", "dDelta", "db"):
            assert rel_err(b[k], a[k]) < 1e-11, (W, k)


def test_window_pin_case_windows_differ(orc):
    """In the slow-decay case adjacent windows differ far above fp32 tolerances."""
    c = window_pin_case(seed=100, T=128, P=8, N=4)
    inp = {k: (np.asarray(v, dtype=np.float64) if isinstance(v, np.ndarray) else v)
           for k, v in make_layer(c).items()}
    prev = None
    for W in (1, 2, 3, 7, 64, 127, 128):
        gr = orc.layer_grad(inp, window=W)
        if prev is not None:
            # W = T adds only the pair (t = T-1, i = 0); h_{-1} = 0 leaves
            # dW_delta unchanged there, but dx (through db_0 and dxdir_0) sees it.
            gap = max(rel_err(gr["dW_delta"], prev[0]), rel_err(gr["dW_B"], prev[1]),
                      rel_err(gr["dx"], prev[2]))
            assert gap > 1e-3, W
        prev = (gr["dW_delta"], gr["dW_B"], gr["dx"])


def test_channel_subset_matches_full(orc):
    inp = _tiny(T=33, P=7, N=4, seed=61)
    full = orc.layer_grad(inp, window=9)
    chans = [5, 0, 3]
    sub = orc.channel_grad(inp, chans, window=9)
    assert rel_err(sub["dDelta"], full["dDelta"][:, chans]) < 1e-14
    assert rel_err(sub["dalpha"], full["dalpha"][chans]) < 1e-14
    assert rel_err(sub["dW_delta_rows"], full["dW_delta"][chans]) < 1e-13
    assert rel_err(sub["y"], full["y"][:, chans]) < 1e-14


# ---------------------------------------------------------------- casts and stack

def test_bf16_cast_matches_torch(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    r = rng.standard_normal(4096) * np.exp(rng.uniform(-20, 20, 4096))
    r[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]  # exact ties
    ours = orc.cast_input(r, "bf16")
    ref = torch.tensor(r, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(orc.cast_input(r, "f32"), r.astype(np.float32).astype(np.float64))


def _stack64(K, T, P, N, seed):
    """Stack inputs with the residual stream kept in double (cast = identity)."""
    c = LayerCase("stack_t", T, P, N, "f32", (), K=K, seed=seed)
    st = make_stack(c)
    st["io"] = "f64"
    st["x"] = np.asarray(st["x"], dtype=np.float64)
    st["g"] = np.asarray(st["g"], dtype=np.float64)
    st["layers"] = [{k: np.asarray(v, dtype=np.float64) for k, v in lay.items()} for lay in st["layers"]]
    return st


@pytest.mark.parametrize("K", [2, 3])
def test_stack_matches_monolithic_autograd(orc, K):
    """Proposition 3: the layer-separated sum equals end-to-end reverse mode."""
    torch = pytest.importorskip("torch")
    st = _stack64(K, T=32, P=6, N=3, seed=70 + K)
    ours = orc.stack_grad(st, window=None)
    ths = [{k: torch.tensor(v, requires_grad=True) for k, v in lay.items()} for lay in st["layers"]]
    x0 = torch.tensor(st["x"], requires_grad=True)
    r = x0
    for th in ths:
        th2 = dict(th, x=r)
        r = r + _torch_forward(th2, 32, 3)
    L = (torch.tensor(st["g"]) * r).sum()
    L.backward()
    for k in range(K):
        for pname, gname in (("W_delta", "dW_delta"), ("W_B", "dW_B"), ("W_C", "dW_C"),
                             ("alpha", "dalpha"), ("delta_bias", "dbias")):
            assert rel_err(ours["layers"][k][gname], ths[k][pname].grad.numpy()) < 1e-11, (k, pname)
    assert rel_err(ours["dx0"], x0.grad.numpy()) < 1e-11


def test_stack_fd_and_g_only_reading_rejected(orc):
    st = _stack64(2, T=12, P=3, N=2, seed=80)
    ours = orc.stack_grad(st, window=None)
    lay0 = st["layers"][0]
    f = lambda: orc.stack_loss(st)
    fd = _fd_grad(f, lay0["W_B"])
    assert rel_err(ours["layers"][0]["dW_B"], fd) < 1e-8
    # Reading "every layer is driven by g alone" gives a different answer.
    g_only = orc.layer_grad(dict(lay0, x=ours["forward"]["x_layers"][0], g=st["g"]), window=None)
    assert rel_err(g_only["dW_B"], fd) > 1e-2


# ---------------------------------------------------------------- normalised layer input

def test_rmsnorm_closed_form(orc):
    rng = np.random.default_rng(91)
    r = rng.standard_normal((6, 40)) * rng.uniform(0.01, 100.0, (6, 1))
    ones = np.ones(40)
    out, rinv = orc.rmsnorm(r, ones, eps=0.0)
    # every row has unit mean square, and scaling a row changes nothing
    assert np.allclose((out ** 2).mean(axis=1), 1.0, rtol=1e-13, atol=0)
    assert np.allclose(orc.rmsnorm(3.7 * r, ones, eps=0.0)[0], out, rtol=1e-13, atol=1e-14)
    assert np.allclose(rinv, 1.0 / np.sqrt((r ** 2).mean(axis=1)), rtol=1e-13)
    # a per-channel scale multiplies the columns; eps damps small rows
    gam = rng.uniform(-2, 2, 40)
    assert np.allclose(orc.rmsnorm(r, gam, eps=0.0)[0], out * gam, rtol=1e-13, atol=1e-14)
    small = np.full((1, 40), 1e-4)
    o, _ = orc.rmsnorm(small, ones, eps=1e-5)
    assert np.allclose(o, 1e-4 / np.sqrt(1e-8 + 1e-5), rtol=1e-13)


def test_rmsnorm_vjp_finite_differences(orc):
    rng = np.random.default_rng(92)
    T, P = 4, 9
    r = rng.standard_normal((T, P))
    gam = rng.uniform(0.5, 1.5, P)
    d = rng.standard_normal((T, P))
    dr, dg = orc.rmsnorm_vjp(r, gam, d)
    f_r = lambda: float(np.sum(d * orc.rmsnorm(r, gam)[0]))
    f_g = lambda: float(np.sum(d * orc.rmsnorm(r, gam)[0]))
    assert rel_err(dr, _fd_grad(f_r, r)) < 1e-8
    assert rel_err(dg, _fd_grad(f_g, gam)) < 1e-8


def test_rmsnorm_vjp_orthogonal_to_input_without_eps(orc):
    # without eps the normalisation is invariant to scaling each row, so the
    # input cotangent of every row is orthogonal to that row
    rng = np.random.default_rng(93)
    r = rng.standard_normal((5, 33))
    dr, _ = orc.rmsnorm_vjp(r, rng.uniform(-1, 1, 33), rng.standard_normal((5, 33)), eps=0.0)
    dots = np.einsum("tp,tp->t", dr, r) / (np.linalg.norm(dr, axis=1) * np.linalg.norm(r, axis=1))
    assert np.abs(dots).max() < 1e-13


@pytest.mark.parametrize("K", [2, 3])
def test_normalised_stack_matches_monolithic_autograd(orc, K):
    """Stack with normalised layer inputs: the oracle's per-layer backward
    (layer VJPs, then the normalisation's VJP) equals end-to-end reverse mode
    through an RMS normalisation written independently in torch."""
    torch = pytest.importorskip("torch")
    T, P, N = 24, 6, 3
    st = _stack64(K, T=T, P=P, N=N, seed=90 + K)
    rng = np.random.default_rng(94 + K)
    for lay in st["layers"]:
        lay["norm_scale"] = rng.uniform(0.5, 1.5, P)
    ours = orc.stack_grad(st, window=None)
    ths = [{k: torch.tensor(v, requires_grad=True) for k, v in lay.items()} for lay in st["layers"]]
    x0 = torch.tensor(st["x"], requires_grad=True)
    r = x0
    for th in ths:
        xin = th["norm_scale"] * r / torch.sqrt((r * r).mean(dim=1, keepdim=True) + orc.NORM_EPS)
        th2 = dict(th, x=xin)
        r = r + _torch_forward(th2, T, N)
    L = (torch.tensor(st["g"]) * r).sum()
    L.backward()
    for k in range(K):
        for pname, gname in (("W_delta", "dW_delta"), ("W_B", "dW_B"), ("W_C", "dW_C"),
                             ("alpha", "dalpha"), ("delta_bias", "dbias"), ("norm_scale", "dnorm_scale")):
            assert rel_err(ours["layers"][k][gname], ths[k][pname].grad.numpy()) < 1e-10, (k, pname)
    assert rel_err(ours["dx0"], x0.grad.numpy()) < 1e-10
