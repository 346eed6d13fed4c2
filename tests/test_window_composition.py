"""The chunk algebra of the windowed adjoint, checked in fp64 on the CPU.

For one channel p and state n the truncated adjoint sum is
  mu_i = sum_{t=i}^{min(T, i+W)-1} g_t c_t prod_{j=i+1}^{t} a_j
(review of "Adjoint sharding for very long context training of state space
models", Core claim: Proposition 2 and truncated adjoint sharding).  The GPU
path splits the sequence into chunks of C tokens and, when W = qC, forms each
chunk's windowed aggregate from two exact ones:
  A_w[k] = A[k] - exp(-alpha sum_{t=t0}^{t0+W-1} s_t) A[k+q],
  A[k]   = sum_{i in chunk k} g_i c_i prod_{j=t0}^{i} a_j        (t0 = kC),
then carries mu across chunks with carry[k-1] = prod_{t in k} a_t carry[k] + A_w[k].
These tests take that identity and the carry from the definition alone (plain
loops, no code of the GPU path) and compare with mu computed directly.
"""
import numpy as np
import pytest


def _case(T, seed, s_scale):
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.2, 1.0, T) * s_scale  # softplus(Delta) > 0
    g = rng.standard_normal(T)
    c = rng.standard_normal(T)
    return s, g, c


def _mu_direct(s, g, c, alpha, W):
    """mu_i from the definition (a_j = exp(-alpha s_j))."""
    T = len(s)
    a = np.exp(-alpha * s)
    mu = np.zeros(T)
    for i in range(T):
        lam = 1.0
        for t in range(i, min(T, i + W)):
            if t > i:
                lam *= a[t]
            mu[i] += g[t] * c[t] * lam
    return mu


def _aggregates(s, g, c, alpha, C, W):
    """Exact chunk aggregates A[k], windowed ones A_w[k] by their definition,
    and the composed ones."""
    T = len(s)
    a = np.exp(-alpha * s)
    K = (T + C - 1) // C
    A = np.zeros(K)
    Aw_def = np.zeros(K)
    for k in range(K):
        t0, t1 = k * C, min(T, k * C + C)
        for i in range(t0, t1):
            w = np.prod(a[t0:i + 1])
            A[k] += g[i] * c[i] * w
            # windowed: a_{t0} * mu^{loc,w}_{t0}; token i's own window term
            # subtracts g_{i+W} c_{i+W} prod_{j=t0}^{i+W} a_j
            Aw_def[k] += g[i] * c[i] * w
            if i + W < T:
                Aw_def[k] -= g[i + W] * c[i + W] * np.prod(a[t0:i + W + 1])
    q = W // C
    Aw_comp = A.copy()
    for k in range(K):
        if k + q < K:
            Aw_comp[k] -= np.exp(-alpha * np.sum(s[k * C:k * C + W])) * A[k + q]
    return A, Aw_def, Aw_comp, a


@pytest.mark.parametrize("T,C,W", [(700, 50, 150), (640, 64, 64), (333, 37, 111), (96, 8, 88)])
@pytest.mark.parametrize("alpha", [0.05, 1.0, 3.0])
def test_composed_aggregates_equal_definition(T, C, W, alpha):
    s, g, c = _case(T, seed=T + C + W, s_scale=0.2)
    _, Aw_def, Aw_comp, _ = _aggregates(s, g, c, alpha, C, W)
    scale = np.max(np.abs(Aw_def))
    assert np.max(np.abs(Aw_comp - Aw_def)) <= 1e-12 * scale


@pytest.mark.parametrize("T,C,W", [(700, 50, 150), (333, 37, 111)])
def test_carry_reproduces_windowed_adjoint(T, C, W):
    alpha = 0.3
    s, g, c = _case(T, seed=7 * T + W, s_scale=0.1)
    _, _, Aw, a = _aggregates(s, g, c, alpha, C, W)
    K = len(Aw)
    # carry[k] = a_{e+1} mu_{e+1} for the last token e of chunk k
    carry = np.zeros(K)
    cin = 0.0
    for k in range(K - 1, -1, -1):
        carry[k] = cin
        cin = np.prod(a[k * C:min(T, k * C + C)]) * cin + Aw[k]
    mu = _mu_direct(s, g, c, alpha, W)
    # mu at the last token of each chunk, walked from the carry: mu_e = g_e c_e + carry
    # minus the token leaving the window, and a_{t0} mu_{t0} = the chunk's aggregate
    # plus the carried-in part
    for k in range(K):
        t0, t1 = k * C, min(T, k * C + C)
        e = t1 - 1
        mu_e = g[e] * c[e] + carry[k]
        if e + W < T:
            mu_e -= g[e + W] * c[e + W] * np.prod(a[e + 1:e + W + 1])
        assert abs(mu_e - mu[e]) <= 1e-11 * np.max(np.abs(mu))
        lhs = a[t0] * mu[t0]
        rhs = Aw[k] + np.prod(a[t0:t1]) * carry[k]
        assert abs(lhs - rhs) <= 1e-11 * np.max(np.abs(mu))
