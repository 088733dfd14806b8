"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each test names the passage it follows.  None re-types the oracle's own
formula: they check printed worked examples (tests/golden), closed forms,
invariants, special cases that reduce to a library routine, and exact
rational arithmetic.
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

from conftest import load_golden
from oracle import chunkwise, exact, kalman
from oracle.recurrence import forward

RNG = np.random.default_rng(1234)


def one(a):
    """[...] -> [1, ...] (a single head)."""
    return np.asarray(a, np.float64)[None]


# --------------------------------------------------------------------------
# Kaczmarz Linear Attention
# --------------------------------------------------------------------------

def test_kla_worked_example():
    """§2.3 teaching example: d=1, decayed state 0, k=2, v=1."""
    g = load_golden("kla_worked_example.json")
    k = one([[2.0]])
    v = one([[1.0]])
    alpha = one([1.0])
    # readout with q = k gives the value read back along the written key
    # GDN with beta = 1
    o, S, _, _ = forward(k, k, v, "gdn", alpha, eta=one([1.0]))
    assert S[0, 0, 0] == g["gdn_beta1"]["S"]
    assert o[0, 0, 0] == g["gdn_beta1"]["readout_Sk"]
    assert 1.0 - o[0, 0, 0] == g["gdn_beta1"]["residual_after"]
    # KLA with eta = 1, eps = 0
    o, S, _, tr = forward(k, k, v, "kla", alpha, eta=one([1.0]), eps=0.0, record=True)
    assert tr["w"][0, 0, 0] / 2.0 == g["kla_eta1"]["beta"]
    assert S[0, 0, 0] == g["kla_eta1"]["S"]
    assert o[0, 0, 0] == g["kla_eta1"]["readout_Sk"]
    # eta = 1/2 halves the residual
    o, S, _, tr = forward(k, k, v, "kla", alpha, eta=one([0.5]), eps=0.0, record=True)
    assert tr["e"][0, 0, 0] == g["kla_eta_half"]["residual_before"]
    assert 1.0 - o[0, 0, 0] == g["kla_eta_half"]["residual_after"]


def test_kla_worked_example_exact():
    """Same example in exact rationals (oracle.exact)."""
    ws, _ = exact.gains([[Fr(2)]], "kla", [Fr(1)], eta=[Fr(1)], eps=Fr(0))
    o, S = exact.token_recurrence([[Fr(2)]], [[Fr(2)]], [[Fr(1)]], ws, [Fr(1)])
    assert S == [[Fr(1, 2)]] and o == [[Fr(1)]]


def _random_head(T, dk, dv, scaled=True, channel=False):
    k = RNG.standard_normal((T, dk))
    if scaled:
        k *= RNG.uniform(0.25, 4.0, size=(T, 1))
    q = RNG.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = RNG.standard_normal((T, dv))
    eta = 1 / (1 + np.exp(-RNG.standard_normal(T)))
    alpha = 1 / (1 + np.exp(-RNG.normal(3, 1, size=(T, dk) if channel else T)))
    S0 = RNG.normal(0, 0.1, size=(dk, dv))
    return q, k, v, eta, alpha, S0


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.3])
def test_kla_contraction_identity(eps):
    """§2.4 Eq. 5: after the write, the residual along the same key shrinks by
    (1 - eta ||k||^2 / (||k||^2 + eps)), for every token."""
    T, dk, dv = 40, 8, 5
    q, k, v, eta, alpha, S0 = _random_head(T, dk, dv)
    for t in range(T):
        _, S_prev, _, _ = forward(one(q[:t]), one(k[:t]), one(v[:t]), "kla", one(alpha[:t]),
                                  eta=one(eta[:t]), eps=eps, S0=one(S0))
        _, S_t, _, tr = forward(one(q[t:t + 1]), one(k[t:t + 1]), one(v[t:t + 1]), "kla",
                                one(alpha[t:t + 1]), eta=one(eta[t:t + 1]), eps=eps,
                                S0=S_prev, record=True)
        e = tr["e"][0, 0]
        n2 = k[t] @ k[t]
        post = v[t] - S_t[0].T @ k[t]
        np.testing.assert_allclose(post, (1 - eta[t] * n2 / (n2 + eps)) * e, rtol=1e-10, atol=1e-12)


def test_kla_projection_is_min_frobenius_change():
    """§2.2 Eqs. 1-2: with eta = 1, eps = 0 the write is the least change of
    the decayed state that satisfies S^T k = v (min-norm lstsq per column)."""
    dk, dv = 7, 4
    for _ in range(5):
        S_prev = RNG.standard_normal((dk, dv))
        k = RNG.standard_normal(dk) * 3
        v = RNG.standard_normal(dv)
        a = 0.8
        _, S, _, _ = forward(one([k]), one([k]), one([v]), "kla", one([a]), eta=one([1.0]),
                             eps=0.0, S0=one(S_prev))
        S_dec = a * S_prev
        delta, *_ = np.linalg.lstsq(k[None, :], (v - S_dec.T @ k)[None, :], rcond=None)
        np.testing.assert_allclose(S[0], S_dec + delta, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S[0].T @ k, v, rtol=1e-12, atol=1e-12)


def test_kla_proximal_form():
    """§2.4 Prop. 1: the relaxed write solves (I + mu k k^T) S = S_dec + mu k v^T
    with mu = eta / ((1 - eta) ||k||^2 + eps)."""
    dk, dv = 6, 3
    for eta, eps in [(0.3, 0.0), (0.7, 1e-3), (0.95, 0.5)]:
        S_prev = RNG.standard_normal((dk, dv))
        k = RNG.standard_normal(dk) * 2
        v = RNG.standard_normal(dv)
        a = 0.9
        _, S, _, _ = forward(one([k]), one([k]), one([v]), "kla", one([a]), eta=one([eta]),
                             eps=eps, S0=one(S_prev))
        mu = eta / ((1 - eta) * (k @ k) + eps)
        rhs = a * S_prev + mu * np.outer(k, v)
        expect = np.linalg.solve(np.eye(dk) + mu * np.outer(k, k), rhs)
        np.testing.assert_allclose(S[0], expect, rtol=1e-11, atol=1e-12)


def test_kla_orthogonal_keys_do_not_interfere():
    """§2.4 cross-key interference: with alpha = eta = 1, eps = 0 and mutually
    orthogonal keys, every stored association reads back exactly."""
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(RNG.standard_normal((dk, dk)))
    K = Qm[:, :n].T * RNG.uniform(0.5, 3, size=(n, 1))
    V = RNG.standard_normal((n, dv))
    _, S, _, _ = forward(one(K), one(K), one(V), "kla", one(np.ones(n)), eta=one(np.ones(n)),
                         eps=0.0, S0=one(RNG.standard_normal((dk, dv))))
    np.testing.assert_allclose(S[0].T @ K.T, V.T, rtol=1e-12, atol=1e-12)


def test_kla_zero_key_keeps_state():
    """§2.4: with eps > 0 a zero key writes nothing (state = decayed state)."""
    dk, dv = 4, 3
    S_prev = RNG.standard_normal((dk, dv))
    _, S, _, tr = forward(one([RNG.standard_normal(dk)]), one([np.zeros(dk)]),
                          one([RNG.standard_normal(dv)]), "kla", one([0.5]), eta=one([0.9]),
                          eps=1e-6, S0=one(S_prev), record=True)
    np.testing.assert_array_equal(S[0], 0.5 * S_prev)
    assert np.all(tr["w"] == 0)


# --------------------------------------------------------------------------
# Preconditioned DeltaNet
# --------------------------------------------------------------------------

def _pgdn_one_step(A0, k, x, mu, eta=1.0, alphaP=1.0, betaP=0.0, S0=None, v=None, a=1.0):
    dk = len(k)
    dv = 2 if v is None else len(v)
    v = np.zeros(dv) if v is None else v
    return forward(one([k]), one([k]), one([v]), "pgdn", one([a]), eta=one([eta]),
                   alphaP=one([alphaP]), betaP=one([betaP]), mu_log=np.array([mu]), x=x,
                   S0=None if S0 is None else one(S0), aux0=one(A0), record=True)


def test_pgdn_scale_worked_example():
    """§2.4 teaching example: mu = log 4, x = 1.5, A = (16, 1) -> B ~ (0.790, 1.266)."""
    g = load_golden("pgdn_scale_example.json")
    _, _, A, tr = _pgdn_one_step(np.array(g["setup"]["A"], float), np.array([1.0, 1.0]),
                                 g["setup"]["x"], math.log(4.0))
    B = tr["B"][0, 0]
    np.testing.assert_array_equal(A[0], g["setup"]["A"])  # betaP = 0, alphaP = 1 keeps A
    np.testing.assert_allclose(B, g["B_printed"], atol=0.5 * 10 ** -g["printed_decimals"])
    assert abs(B[0] * B[1] - 1.0) < 1e-14  # r is antisymmetric about mu -> B1 B2 = 1
    np.testing.assert_allclose(tr["w"][0, 0], B)  # w = eta B * k with k = 1


def test_pgdn_scale_uses_current_statistic():
    """§2.4, Eq. 9 and the three changes listed after it: the write scale B_t
    is formed from the current statistic A_t, which already holds k_t * k_t.
    Two tokens chosen so that A_1 = (16, 1) is the teaching example's
    statistic (B_1 printed on the page) and A_2 = (4, 4) sits at the centre
    mu = log 4 (B_2 = 1 exactly); a scale formed from A_{t-1} differs in
    both tokens."""
    g = load_golden("pgdn_current_statistic_example.json")
    su = g["setup"]
    toks = su["tokens"]
    k = np.sqrt(np.array([t["k_squared"] for t in toks], float))
    T = len(toks)
    _, _, A, tr = forward(one(k), one(k), one(np.zeros((T, 2))), "pgdn", one(np.ones(T)),
                          eta=one(np.full(T, su["eta"])),
                          alphaP=one([t["alphaP"] for t in toks]),
                          betaP=one([t["betaP"] for t in toks]), mu_log=np.array([math.log(4.0)]),
                          x=su["x"], aux0=one(su["A0"]), record=True)
    np.testing.assert_allclose(tr["A"][0], g["A"], rtol=1e-14)
    np.testing.assert_allclose(A[0], g["A"][-1], rtol=1e-14)
    B = tr["B"][0]
    half_ulp = 0.5 * 10 ** -g["printed_decimals"]
    np.testing.assert_allclose(B, g["B_printed"], atol=half_ulp)
    np.testing.assert_allclose(B[1], [1.0, 1.0], rtol=0, atol=1e-15)
    # the scale from the previous statistic is far from what the oracle forms
    stale = np.asarray(g["B_from_previous_statistic"], float)
    assert np.abs(B - stale).max(axis=1).min() > 0.1
    # w_t = eta B_t * k_t (Eq. 9 with the raw key scaled per channel)
    np.testing.assert_allclose(tr["w"][0], su["eta"] * B * k, rtol=1e-14)


def test_pgdn_scale_bounds():
    """§2.4: B in [1/x, x] for every A > 0; for unit k, k^T k~ in [1/x, x] (§2.7)."""
    dk, x = 64, 1.5
    A0 = np.exp(RNG.uniform(-30, 30, size=dk))
    k = RNG.standard_normal(dk)
    k /= np.linalg.norm(k)
    _, _, _, tr = _pgdn_one_step(A0, k, x, 0.7, betaP=0.5, alphaP=0.9)
    B = tr["B"][0, 0]
    assert np.all(B >= 1 / x) and np.all(B <= x)
    ktk = k @ tr["w"][0, 0]
    assert 1 / x <= ktk <= x


def test_pgdn_x1_reduces_to_gdn():
    """§2.7: x = 1 gives B = 1, i.e. the GDN write."""
    T, dk, dv = 20, 6, 4
    q, k, v, eta, alpha, S0 = _random_head(T, dk, dv, scaled=False)
    kw = dict(eta=one(eta), S0=one(S0))
    o1, S1, _, _ = forward(one(q), one(k), one(v), "pgdn", one(alpha), alphaP=one(np.full(T, .9)),
                           betaP=one(np.full(T, .5)), mu_log=np.array([0.3]), x=1.0, **kw)
    o2, S2, _, _ = forward(one(q), one(k), one(v), "gdn", one(alpha), **kw)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=1e-13, atol=1e-13)


def test_pgdn_statistic_is_cumulative_sum():
    """§2.3: with alphaP = betaP = 1 the statistic is A_0 + running sum of k*k,
    including the current token."""
    T, dk = 30, 5
    k = RNG.standard_normal((T, dk))
    A0 = RNG.uniform(0.5, 2, size=dk)
    _, _, _, tr = forward(one(k), one(k), one(np.zeros((T, 2))), "pgdn", one(np.ones(T)),
                          eta=one(np.ones(T)), alphaP=one(np.ones(T)), betaP=one(np.ones(T)),
                          mu_log=np.array([0.0]), x=1.5, aux0=one(A0), record=True)
    np.testing.assert_allclose(tr["A"][0], A0 + np.cumsum(k * k, axis=0), rtol=1e-13)


def test_pgdn_single_step_spectrum():
    """§2.7: one step maps S -> alpha (I - beta k~ k^T) S; its eigenvalues are
    alpha (d-1 times) and alpha (1 - beta k^T k~), with right eigenvector k~
    and left eigenvector k (the residual uses the raw key)."""
    d, a, beta = 6, 0.9, 0.8
    k = RNG.standard_normal(d)
    k /= np.linalg.norm(k)
    A0 = np.exp(RNG.uniform(-2, 3, size=d))
    _, S1, _, tr = _pgdn_one_step(A0, k, 1.5, 0.4, eta=beta, alphaP=0.95, betaP=0.5,
                                  S0=np.eye(d), v=np.zeros(d), a=a)
    Tm = S1[0]  # image of the identity = the transition matrix
    kt = tr["w"][0, 0] / beta  # k~ = B * k
    lam = a * (1 - beta * (k @ kt))
    ev = np.sort(np.linalg.eigvals(Tm).real)
    expect = np.sort(np.r_[np.full(d - 1, a), lam])
    np.testing.assert_allclose(ev, expect, atol=1e-12)
    np.testing.assert_allclose(Tm @ kt, lam * kt, atol=1e-12)
    np.testing.assert_allclose(k @ Tm, lam * k, atol=1e-12)


def test_ridge_equals_exact_atk():
    """§2.2 Thm 3.1: DeltaNet with the exact ATK write key (Sherman-Morrison
    inverse Gram, P_0 = I/lambda) and no decay reads out the ridge solution
    at every step."""
    T, dk, dv, lam = 25, 6, 4, 0.7
    K = RNG.standard_normal((T, dk))
    V = RNG.standard_normal((T, dv))
    Qr = RNG.standard_normal((T, dk))
    W, _ = kalman.atk_write_vectors(K, lam)
    o, S, _, _ = forward(one(Qr), one(K), one(V), "explicit", one(np.ones(T)), w=one(W))
    np.testing.assert_allclose(S[0], kalman.ridge(K, V, lam), rtol=1e-10, atol=1e-12)
    for t in range(T):
        np.testing.assert_allclose(o[0, t], kalman.ridge(K[:t + 1], V[:t + 1], lam).T @ Qr[t],
                                   rtol=1e-9, atol=1e-11)


def test_diagonal_counterexample():
    """§2.3: lambda = 1, k = v = (1, 1): exact ATK gives S_1 = 1/3 11^T,
    the diagonal ATQ readout gives 1/2 11^T."""
    g = load_golden("pdn_diagonal_counterexample.json")
    k = np.array([g["setup"]["k1"]], float)
    v = np.array([g["setup"]["v1"]], float)
    W, _ = kalman.atk_write_vectors(k, g["setup"]["lambda"])
    _, S, _, _ = forward(one(k), one(k), one(v), "explicit", one([1.0]), w=one(W))
    np.testing.assert_allclose(S[0], float(Fr(g["atk_S1_entry"])) * np.ones((2, 2)), rtol=1e-15)
    A = g["setup"]["lambda"] + k[0] * k[0]
    atq = np.outer(k[0], v[0]) / A[:, None]  # C diag(1/A), d_k x d_v orientation
    np.testing.assert_allclose(atq, float(Fr(g["diagonal_atq_S1_entry"])) * np.ones((2, 2)))


# --------------------------------------------------------------------------
# Kalman Delta Networks
# --------------------------------------------------------------------------

def _kdn(k, v, alpha, omega, r, mu_info, p0, S0=None, q=None):
    q = k if q is None else q
    return forward(one(q), one(k), one(v), "kdn", one(alpha), omega=one(omega), r=one(r),
                   mu_info=mu_info, aux0=one(p0), S0=None if S0 is None else one(S0), record=True)


def test_kdn_scalar_gains():
    """§2.2 teaching example: k = r = 1, predicted variance 9 -> gain 0.9;
    0.1 -> about 0.0909."""
    g = load_golden("kdn_gain_example.json")
    for case in g["cases"]:
        _, _, _, tr = _kdn(np.array([[1.0]]), np.array([[0.0]]), np.array([[1.0]]),
                           np.array([[0.0]]), np.array([1.0]), 1.0,
                           np.array([case["predicted_variance"]], float))
        assert tr["p_hat"][0, 0, 0] == case["predicted_variance"]
        assert abs(tr["w"][0, 0, 0] - case["gain_printed"]) <= 0.5 * 10 ** -case["printed_decimals"]


def test_kdn_repeated_observation_exact():
    """§2.2: D = 1, Omega = 0, initial variance 1, repeated k = r = 1:
    variance 1/(n+1), and the mean is the running average with one prior
    pseudo-observation at 0 — exact in rationals."""
    n = 12
    vs = [[Fr(int(x)), Fr(int(y), 3)] for x, y in RNG.integers(-9, 9, size=(n, 2))]
    k = [[Fr(1)]] * n
    ws, ps = exact.gains(k, "kdn", [Fr(1)] * n, omega=[[Fr(0)]] * n, r=[Fr(1)] * n,
                         mu_info=Fr(1), p0=[Fr(1)])
    _, S = exact.token_recurrence(k, k, vs, ws, [Fr(1)] * n)
    for i, p in enumerate(ps):
        assert p == [Fr(1, i + 2)]
    assert S[0] == [sum((v[j] for v in vs), Fr(0)) / (n + 1) for j in range(2)]


def test_kdn_onehot_keys_equal_dense_kalman():
    """§2.4: with diagonal D, Omega and one-hot keys the exact posterior stays
    diagonal, so diagonal KDN (mu = 1) equals the dense textbook filter."""
    T, dk, dv = 30, 4, 3
    idx = RNG.integers(0, dk, size=T)
    k = np.zeros((T, dk))
    k[np.arange(T), idx] = RNG.uniform(0.3, 3, size=T)
    v = RNG.standard_normal((T, dv))
    alpha = RNG.uniform(0.6, 1.0, size=(T, dk))
    omega = RNG.uniform(0.0, 0.3, size=(T, dk))
    r = RNG.uniform(0.2, 2.0, size=T)
    p0 = RNG.uniform(0.5, 2, size=dk)
    S0 = RNG.standard_normal((dk, dv))
    _, S, p, tr = _kdn(k, v, alpha, omega, r, 1.0, p0, S0=S0)
    D = np.stack([np.diag(a) for a in alpha])
    Om = np.stack([np.diag(w) for w in omega])
    S_k, P_k, kap = kalman.dense_kalman(k, v, D, Om, r, S0, np.diag(p0))
    np.testing.assert_allclose(S[0], S_k, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(p[0], np.diag(P_k), rtol=1e-12)
    np.testing.assert_allclose(P_k, np.diag(np.diag(P_k)), atol=1e-15)
    np.testing.assert_allclose(tr["w"][0], kap, rtol=1e-12, atol=1e-14)


def test_dense_kalman_is_bayesian_ridge():
    """Kalman Delta Networks §2.1-2.2 with D = I, Omega = 0: the filter mean is
    the posterior mean of Bayesian linear regression, i.e. ridge regression
    with lambda = r / p0 (pins the textbook filter itself)."""
    T, dk, dv, r, p0 = 40, 5, 3, 0.4, 2.0
    K = RNG.standard_normal((T, dk))
    V = RNG.standard_normal((T, dv))
    eye = np.stack([np.eye(dk)] * T)
    S, _, _ = kalman.dense_kalman(K, V, eye, 0 * eye, np.full(T, r), np.zeros((dk, dv)),
                                  p0 * np.eye(dk))
    np.testing.assert_allclose(S, kalman.ridge(K, V, r / p0), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mu_key", ["directional_variance_projected_mu1_printed",
                                    "directional_variance_projected_mu128_printed"])
def test_kdn_uniform_energy_example(mu_key):
    """§2.5: m = 128 channels with k_i^2 = 1/m and p_hat = r = 1: the projected
    directional variance is about 0.9922 for mu = 1 and 0.5 for mu = 128;
    the exact value is r p / (r + p) = 0.5."""
    g = load_golden("kdn_uniform_energy.json")
    m = g["setup"]["m"]
    mu = 1.0 if "mu1_" in mu_key else float(m)
    k = np.full((1, m), 1 / math.sqrt(m))
    _, _, p, tr = _kdn(k, np.zeros((1, 2)), np.ones((1, m)), np.zeros((1, m)), np.ones(1), mu,
                       np.ones(m))
    assert np.all(tr["p_hat"] == 1.0)
    V_proj = float(k[0] ** 2 @ p[0])
    assert abs(V_proj - g[mu_key]) <= 0.5 * 10 ** -g["printed_decimals"]
    # exact directional variance of the dense posterior (P_hat^-1 + k k^T / r)^-1
    P_exact = np.linalg.inv(np.eye(m) + np.outer(k[0], k[0]))
    assert abs(k[0] @ P_exact @ k[0] - g["directional_variance_exact"]) < 1e-12


def test_kdn_effective_gain_in_unit_interval():
    """Kalman Delta Networks §2.2: beta_eff = k^T kappa lies in [0, 1)."""
    T, dk, dv = 200, 16, 4
    q, k, v, _, alpha, S0 = _random_head(T, dk, dv, channel=True)
    omega = np.log1p(np.exp(RNG.normal(-3, 1, size=(T, dk))))
    r = np.log1p(np.exp(RNG.standard_normal(T)))
    _, _, _, tr = _kdn(k, v, alpha, omega, r, 1.0, np.ones(dk), S0=S0, q=q)
    be = np.einsum("td,td->t", k, tr["w"][0])
    assert np.all(be >= 0) and np.all(be < 1)


def test_kdn_variance_matches_mobius_scan():
    """§2.6 Eqs. 32-37: the variance recurrence is a Moebius map; prefix
    products of M_t = [[a^2, w], [u a^2, 1 + u w]] applied to (p_0, 1),
    rescaled by max-abs, give p_t = n_t / d_t."""
    T, dk, mu = 300, 8, 3.0
    k = RNG.standard_normal((T, dk)) * 2
    alpha = RNG.uniform(0.5, 1.0, size=(T, dk))
    omega = RNG.uniform(0.0, 0.5, size=(T, dk))
    r = RNG.uniform(0.05, 2.0, size=T)
    p0 = RNG.uniform(0.5, 2, size=dk)
    _, _, _, tr = _kdn(k, np.zeros((T, 1)), alpha, omega, r, mu, p0)
    u = mu / r[:, None] * k * k
    a2 = alpha * alpha
    for i in range(dk):
        Pm = np.eye(2)
        for t in range(T):
            Mt = np.array([[a2[t, i], omega[t, i]], [u[t, i] * a2[t, i], 1 + u[t, i] * omega[t, i]]])
            Pm = Mt @ Pm
            Pm /= np.abs(Pm).max()
            nd = Pm @ np.array([p0[i], 1.0])
            assert abs(nd[0] / nd[1] - tr["p"][0, t, i]) <= 1e-12 * tr["p"][0, t, i]


# --------------------------------------------------------------------------
# Isotropic KDN (Kalman Delta Networks §2.7, Eq. 40)
# --------------------------------------------------------------------------

def _iso(k, v, alpha, omega, r, mu_info, b0, S0=None, q=None):
    q = k if q is None else q
    return forward(one(q), one(k), one(v), "kdn_iso", one(alpha), omega=one(omega), r=one(r),
                   mu_info=mu_info, aux0=np.array([b0], float),
                   S0=None if S0 is None else one(S0), record=True)


@pytest.mark.parametrize("channel", [False, True])
def test_kdn_iso_one_channel_equals_diagonal(channel):
    """§2.7: with a single key channel the isotropic and the diagonal variance
    are the same number, so both variants give the same gains, variances,
    outputs and state (ties the isotropic branch to the diagonal pins)."""
    T, dv = 80, 3
    k = RNG.standard_normal((T, 1)) * 2
    q = RNG.standard_normal((T, 1))
    v = RNG.standard_normal((T, dv))
    alpha = RNG.uniform(0.5, 1.0, size=(T, 1) if channel else T)
    omega = RNG.uniform(0.0, 0.4, size=T)
    r = RNG.uniform(0.1, 2.0, size=T)
    S0 = RNG.standard_normal((1, dv))
    o_i, S_i, b, tr_i = _iso(k, v, alpha, omega, r, 1.7, 1.3, S0=S0, q=q)
    o_d, S_d, p, tr_d = _kdn(k, v, alpha if channel else alpha[:, None], omega[:, None], r, 1.7,
                             np.array([1.3]), S0=S0, q=q)
    np.testing.assert_allclose(tr_i["w"], tr_d["w"], rtol=1e-13)
    np.testing.assert_allclose(tr_i["p"], tr_d["p"][..., 0], rtol=1e-13)
    np.testing.assert_allclose(o_i, o_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_i, S_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b, p[:, 0], rtol=1e-13)


def test_kdn_iso_steps_are_kalman_steps_with_the_two_projections():
    """§2.7: prediction projects D (b I) D^T + omega I to the isotropic matrix
    with the same trace; the gain is the exact Kalman gain of that isotropic
    prediction (textbook filter); the reverse-KL projection of the exact
    posterior keeps the harmonic mean of its eigenvalues (mu = 1)."""
    T, dk, dv = 25, 6, 2
    k = RNG.standard_normal((T, dk)) * RNG.uniform(0.3, 3, size=(T, 1))
    v = RNG.standard_normal((T, dv))
    alpha = RNG.uniform(0.6, 1.0, size=(T, dk))
    omega = RNG.uniform(0.0, 0.3, size=T)
    r = RNG.uniform(0.2, 2.0, size=T)
    _, _, _, tr = _iso(k, v, alpha, omega, r, 1.0, 0.8)
    b = 0.8
    for t in range(T):
        P_hat = np.diag(alpha[t]) @ (b * np.eye(dk)) @ np.diag(alpha[t]) + omega[t] * np.eye(dk)
        b_hat = np.trace(P_hat) / dk
        assert abs(tr["p_hat"][0, t] - b_hat) <= 1e-14 * b_hat
        _, P_post, kap = kalman.dense_kalman(k[t:t + 1], v[t:t + 1], np.eye(dk)[None],
                                             np.zeros((1, dk, dk)), r[t:t + 1], np.zeros((dk, dv)),
                                             b_hat * np.eye(dk))
        np.testing.assert_allclose(tr["w"][0, t], kap[0], rtol=1e-12, atol=1e-15)
        eig = np.linalg.eigvalsh((P_post + P_post.T) / 2)
        b = dk / np.sum(1.0 / eig)
        assert abs(tr["p"][0, t] - b) <= 1e-11 * b


def test_kdn_iso_repeated_observation_exact():
    """§2.7: with mu = d_k and a unit key the information term is 1 / r; with
    D = 1, omega = 0, r = 1 and b_0 = 1 the variance is 1/(n+1) and the read
    along the key is the running mean with one prior pseudo-observation at 0
    (exact in rationals)."""
    n, dk = 10, 4
    key = [Fr(3, 5), Fr(4, 5), Fr(0), Fr(0)]
    vs = [[Fr(int(x)), Fr(int(y), 7)] for x, y in RNG.integers(-9, 9, size=(n, 2))]
    k = [key] * n
    ws, bs = exact.gains(k, "kdn_iso", [Fr(1)] * n, omega=[Fr(0)] * n, r=[Fr(1)] * n,
                         mu_info=Fr(dk), p0=[Fr(1)])
    _, S = exact.token_recurrence(k, k, vs, ws, [Fr(1)] * n)
    for i, b in enumerate(bs):
        assert b == [Fr(1, i + 2)]
    read = [sum((S[d][j] * key[d] for d in range(dk)), Fr(0)) for j in range(2)]
    assert read == [sum((v[j] for v in vs), Fr(0)) / (n + 1) for j in range(2)]


def test_kdn_iso_effective_gain_in_unit_interval():
    """§2.7 with §2.2: beta_eff = k^T kappa = b_hat ||k||^2 / (r + b_hat ||k||^2)
    lies in [0, 1) for any positive noise."""
    T, dk, dv = 200, 16, 4
    q, k, v, _, alpha, S0 = _random_head(T, dk, dv, channel=True)
    omega = np.log1p(np.exp(RNG.normal(-3, 1, size=T)))
    r = np.log1p(np.exp(RNG.standard_normal(T)))
    _, _, _, tr = _iso(k, v, alpha, omega, r, 1.0, 1.0, S0=S0, q=q)
    be = np.einsum("td,td->t", k, tr["w"][0])
    assert np.all(be >= 0) and np.all(be < 1)


# --------------------------------------------------------------------------
# Chunkwise form == recurrence (Kaczmarz Linear Attention §2.5;
# Preconditioned DeltaNet §2.6; Kalman Delta Networks §2.6)
# --------------------------------------------------------------------------

def _rat(x, den=8):
    return Fr(int(round(x * den)), den)


@pytest.mark.parametrize("gain", ["kla", "gdn", "kdn", "kdn_iso", "explicit"])
@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("T,C", [(1, 1), (5, 2), (9, 4), (13, 4)])
def test_chunk_form_equals_recurrence_exactly(gain, channel, T, C):
    dk, dv = 3, 2
    rnd = lambda *s: RNG.uniform(-1, 1, size=s)
    k = [[_rat(x) for x in row] for row in rnd(T, dk) * 2]
    q = [[_rat(x) for x in row] for row in rnd(T, dk)]
    v = [[_rat(x) for x in row] for row in rnd(T, dv)]
    S0 = [[_rat(x) for x in row] for row in rnd(dk, dv)]
    if channel:
        alpha = [[Fr(int(x), 8) for x in row] for row in RNG.integers(4, 9, size=(T, dk))]
    else:
        alpha = [Fr(int(x), 8) for x in RNG.integers(4, 9, size=T)]
    kw = dict(eta=[Fr(int(x), 4) for x in RNG.integers(1, 5, size=T)], eps=Fr(1, 100),
              omega=[[Fr(int(x), 16) for x in row] for row in RNG.integers(0, 4, size=(T, dk))],
              r=[Fr(int(x), 4) for x in RNG.integers(1, 8, size=T)], mu_info=Fr(3, 2),
              w=[[_rat(x) for x in row] for row in rnd(T, dk)], p0=[Fr(1)] * dk)
    if gain == "kdn_iso":  # scalar process noise and one variance per head
        kw["omega"] = [Fr(int(x), 16) for x in RNG.integers(0, 4, size=T)]
        kw["p0"] = [Fr(5, 4)]
    ws, _ = exact.gains(k, gain, alpha, **kw)
    o_rec, S_rec = exact.token_recurrence(q, k, v, ws, alpha, S0)
    o_chk, S_chk = exact.chunkwise(q, k, v, ws, alpha, C, S0)
    assert o_rec == o_chk and S_rec == S_chk
    # the fp64 oracle agrees with exact arithmetic
    f = lambda M: np.array([[float(x) for x in row] for row in M])
    fa = lambda a: np.array([[float(x) for x in row] for row in a]) if channel else \
        np.array([float(x) for x in a])
    om = [float(x) for x in kw["omega"]] if gain == "kdn_iso" else f(kw["omega"])
    o64, S64, _, _ = forward(one(f(q)), one(f(k)), one(f(v)), gain, one(fa(alpha)),
                             eta=one([float(x) for x in kw["eta"]]), eps=0.01,
                             omega=one(om), r=one([float(x) for x in kw["r"]]),
                             mu_info=1.5, w=one(f(kw["w"])), S0=one(f(S0)),
                             aux0=np.array([1.25]) if gain == "kdn_iso" else None)
    np.testing.assert_allclose(o64[0], f(o_rec), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S64[0], f(S_rec), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("gain", ["kla", "gdn", "pgdn", "kdn", "kdn_iso"])
def test_chunk_form_equals_recurrence_fp64(gain):
    N, T, dk, dv, C = 3, 150, 16, 12, 64
    channel = gain in ("kdn", "kdn_iso")
    heads = [_random_head(T, dk, dv, scaled=gain in ("kla", "kdn", "kdn_iso"), channel=channel)
             for _ in range(N)]
    q, k, v, eta, alpha, S0 = (np.stack(x) for x in zip(*heads))
    kw = dict(eta=eta, eps=1e-6, alphaP=1 / (1 + np.exp(-RNG.normal(2, 1, (N, T)))),
              betaP=1 / (1 + np.exp(-RNG.normal(2, 1, (N, T)))), mu_log=np.full(N, math.log(4)),
              x=1.5, omega=np.log1p(np.exp(RNG.normal(-3, 1, (N, T) if gain == "kdn_iso" else (N, T, dk)))),
              r=np.log1p(np.exp(RNG.standard_normal((N, T)))), mu_info=1.0)
    o, S, _, tr = forward(q, k, v, gain, alpha, S0=S0, record=True, **kw)
    o2, S2 = chunkwise.forward(q, k, v, tr["w"], alpha, C, S0=S0)
    scale = np.abs(o).max()
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-11 * scale)
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-11 * np.abs(S).max())


@pytest.mark.parametrize("gain", ["kla", "pgdn", "kdn", "kdn_iso"])
def test_resume_equals_single_pass(gain):
    """Tokenwise and chunkwise computation share one recurrence: splitting
    the sequence and carrying (S, aux) reproduces one pass."""
    T, dk, dv, T1 = 90, 8, 6, 37
    channel = gain in ("kdn", "kdn_iso")
    q, k, v, eta, alpha, S0 = _random_head(T, dk, dv, channel=channel)
    kw = dict(eta=eta, eps=1e-6, alphaP=np.full(T, 0.9), betaP=np.full(T, 0.6), x=1.5,
              omega=np.full(T, 0.05) if gain == "kdn_iso" else np.full((T, dk), 0.05),
              r=np.full(T, 0.7), mu_info=2.0)
    full = forward(one(q), one(k), one(v), gain, one(alpha), mu_log=np.array([1.0]), S0=one(S0),
                   **{n: one(a) if isinstance(a, np.ndarray) else a for n, a in kw.items()})
    cut = lambda a, s: one(a[s]) if isinstance(a, np.ndarray) else a
    a1 = forward(one(q[:T1]), one(k[:T1]), one(v[:T1]), gain, one(alpha[:T1]),
                 mu_log=np.array([1.0]), S0=one(S0), **{n: cut(a, slice(0, T1)) for n, a in kw.items()})
    a2 = forward(one(q[T1:]), one(k[T1:]), one(v[T1:]), gain, one(alpha[T1:]),
                 mu_log=np.array([1.0]), S0=a1[1], aux0=a1[2],
                 **{n: cut(a, slice(T1, None)) for n, a in kw.items()})
    np.testing.assert_allclose(np.concatenate([a1[0], a2[0]], axis=1), full[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a2[1], full[1], rtol=1e-12, atol=1e-12)
