"""Pins of the fp64 backward oracle (oracle/backward.py): its gradients
against central finite differences of the forward oracle
(oracle/recurrence.py), element by element, for every gain and decay mode,
plus closed forms of one token."""
import numpy as np
import pytest

from oracle.backward import backward
from oracle.recurrence import forward

RNG = np.random.default_rng(777)


def _inputs(gain, channel, N=2, T=5, dk=3, dv=2):
    rng = np.random.default_rng(abs(hash((gain, channel))) % 2**32)
    f = {}
    f["q"] = rng.standard_normal((N, T, dk))
    f["k"] = rng.standard_normal((N, T, dk)) * (0.6 if gain in ("gdn", "pgdn") else 1.0)
    f["v"] = rng.standard_normal((N, T, dv))
    f["alpha"] = rng.uniform(0.5, 0.95, size=(N, T, dk) if channel else (N, T))
    f["S0"] = rng.normal(0, 0.5, size=(N, dk, dv))
    kw = {}
    if gain in ("kla", "gdn", "pgdn"):
        f["eta"] = rng.uniform(0.2, 0.9, size=(N, T))
    if gain == "kla":
        kw["eps"] = 0.3
    if gain == "pgdn":
        f["alphaP"] = rng.uniform(0.5, 0.9, size=(N, T))
        f["betaP"] = rng.uniform(0.2, 0.8, size=(N, T))
        f["mu_log"] = np.array([2.5, -2.5])[:N]  # |log A - mu| stays away from the softsign kink
        f["aux0"] = rng.uniform(0.5, 2.0, size=(N, dk))
        kw["x"] = 1.5
    if gain == "kdn":
        f["omega"] = rng.uniform(0.05, 0.4, size=(N, T, dk))
        f["r"] = rng.uniform(0.5, 2.0, size=(N, T))
        f["aux0"] = rng.uniform(0.5, 2.0, size=(N, dk))
        kw["mu_info"] = 1.5
    if gain == "kdn_iso":
        f["omega"] = rng.uniform(0.05, 0.4, size=(N, T))
        f["r"] = rng.uniform(0.5, 2.0, size=(N, T))
        f["aux0"] = rng.uniform(0.5, 2.0, size=(N,))
        kw["mu_info"] = 1.5
    if gain == "explicit":
        f["w"] = rng.standard_normal((N, T, dk)) * 0.5
    has_aux = gain in ("pgdn", "kdn", "kdn_iso")
    cot = {"dO": rng.standard_normal((N, T, dv)), "dS_T": rng.standard_normal((N, dk, dv)),
           "daux_T": (rng.standard_normal((N,) if gain == "kdn_iso" else (N, dk)) if has_aux else None)}
    return f, kw, cot


def _loss(gain, f, kw, cot):
    args = {n: a for n, a in f.items() if n not in ("q", "k", "v", "alpha")}
    o, S, aux, _ = forward(f["q"], f["k"], f["v"], gain, f["alpha"], **args, **kw)
    L = np.sum(o * cot["dO"]) + np.sum(S * cot["dS_T"])
    if cot["daux_T"] is not None:
        L += np.sum(np.asarray(aux).reshape(cot["daux_T"].shape) * cot["daux_T"])
    return L


CASES = [("kla", False), ("kla", True), ("gdn", False), ("gdn", True), ("pgdn", False), ("pgdn", True),
         ("kdn", True), ("kdn", False), ("kdn_iso", True), ("kdn_iso", False), ("explicit", False)]


@pytest.mark.parametrize("gain,channel", CASES)
def test_backward_matches_central_differences(gain, channel):
    """Every element of every input: (L(x + h) - L(x - h)) / 2h against the
    reverse sweep, h = 1e-6 (fp64)."""
    f, kw, cot = _inputs(gain, channel)
    args = {n: a for n, a in f.items() if n not in ("q", "k", "v", "alpha")}
    g = backward(f["q"], f["k"], f["v"], gain, f["alpha"], cot["dO"], dS_T=cot["dS_T"],
                 daux_T=cot["daux_T"], **args, **kw)
    h = 1e-6
    for name, arr in f.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(gain, f, kw, cot)
            arr[idx] = old - h
            lm = _loss(gain, f, kw, cot)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        got = np.asarray(g[name]).reshape(arr.shape)
        scale = max(1.0, np.abs(fd).max())
        np.testing.assert_allclose(got, fd, rtol=0, atol=2e-6 * scale, err_msg=f"{gain} d{name}")


def test_one_token_gdn_closed_form():
    """One GDN token, d_k = d_v = 1: o = S q with S = a S0 + eta k (v - a S0 k),
    so dL/dv = eta k q dO, dL/deta = k (v - a S0 k) q dO and
    dL/dS0 = a (1 - eta k^2) q dO, written out by hand."""
    a, S0, eta, k, v, q, dO = 0.8, 0.7, 0.6, 1.3, -0.4, 0.9, 1.7
    g = backward(np.array([[[q]]]), np.array([[[k]]]), np.array([[[v]]]), "gdn", np.array([[a]]),
                 np.array([[[dO]]]), eta=np.array([[eta]]), S0=np.array([[[S0]]]))
    e = v - a * S0 * k
    assert np.isclose(g["v"][0, 0, 0], eta * k * q * dO, rtol=1e-14)
    assert np.isclose(g["eta"][0, 0], k * e * q * dO, rtol=1e-14)
    assert np.isclose(g["S0"][0, 0, 0], a * (1 - eta * k * k) * q * dO, rtol=1e-14)
    assert np.isclose(g["q"][0, 0, 0], (a * S0 + eta * k * e) * dO, rtol=1e-14)
