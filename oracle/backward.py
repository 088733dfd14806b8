"""Gradients of the gated delta-rule recurrence by a reverse sweep, in fp64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): imported by tests, never
by the product.

Training runs the same recurrence as oracle.recurrence.forward and
backpropagates through it (Preconditioned DeltaNet §2.5: training uses the
equivalent chunk form with outer backpropagation; Kalman Delta Networks,
Appendix D: the gain scan and the memory recurrence are both differentiated).
This module is the plain definition of those gradients: for the scalar loss

    L = sum_t <dO_t, o_t> + <dS_T, S_T> + <daux_T, aux_T>

it returns dL/d(input) for every input of the forward pass, by walking the
tokens backwards through the steps of recurrence.forward, each step's
derivative written out by hand from its formula:

  readout     o = S^T q                 dq = S dO,   dS += q dO^T
  write       S = S_dec + w e^T         dw = dS e,   de = dS^T w,  dS_dec = dS
  residual    e = v - S_dec^T k         dv = de,     dk -= S_dec de,
                                        dS_dec -= k de^T
  decay       S_dec = a S_{t-1}         dS_{t-1} = a dS_dec,  da += <dS_dec, S_{t-1}>
                                        (per row for channel decay)
  gain        w = gain(k, gates, aux_{t-1}) -> gradients of k, the gates and
              aux_{t-1} (the per-gain derivations are in _gain_backward)

The forward values every step needs (S_{t-1}, e_t, the gain's intermediate
values) are recomputed here by the same formulas as recurrence.forward, in
fp64; nothing is shared with the GPU path.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def backward(q, k, v, gain, alpha, dO, *, eta=None, eps=0.0, alphaP=None, betaP=None,
             mu_log=None, x=None, omega=None, r=None, mu_info=None, w=None, S0=None, aux0=None,
             dS_T=None, daux_T=None) -> Dict[str, Optional[np.ndarray]]:
    """Gradients of L (module docstring) for N heads.

    Arguments as recurrence.forward (shapes [N, T, ...]; mu_log [N]), plus
    dO [N, T, dv], dS_T [N, dk, dv] (None: 0) and daux_T (None: 0; [N, dk] for
    pgdn / kdn, [N] for kdn_iso).  Returns a dict with the gradient of every
    input the gain uses: q, k, v, alpha, S0, aux0 and (by gain) eta, alphaP,
    betaP, mu_log, omega, r, w.  eps, x and mu_info are constants.
    """
    q, k, v, alpha, dO = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(dO)
    N, T, dk = k.shape
    dv = v.shape[-1]
    channel = alpha.ndim == 3
    eta, alphaP, betaP, mu_log = _f64(eta), _f64(alphaP), _f64(betaP), _f64(mu_log)
    omega, r, w_in = _f64(omega), _f64(r), _f64(w)
    has_aux = gain in ("pgdn", "kdn", "kdn_iso")

    # ---- forward, keeping what the reverse sweep needs
    S = np.zeros((N, dk, dv)) if S0 is None else _f64(S0).copy()
    aux = None
    if gain in ("pgdn", "kdn"):
        aux = np.ones((N, dk)) if aux0 is None else _f64(aux0).copy()
    elif gain == "kdn_iso":
        aux = np.ones(N) if aux0 is None else _f64(aux0).reshape(N).copy()
    Sprev, Es, Ws, auxprev, cache = [], [], [], [], []
    for t in range(T):
        kt = k[:, t]
        a = alpha[:, t] if channel else alpha[:, t][:, None]
        S_dec = a[:, :, None] * S
        auxprev.append(None if aux is None else aux.copy())
        c = {}
        if gain == "kla":
            n = np.sum(kt * kt, axis=1)
            c["n"] = n
            wt = (eta[:, t] / (n + eps))[:, None] * kt
        elif gain == "gdn":
            wt = eta[:, t][:, None] * kt
        elif gain == "pgdn":
            A = alphaP[:, t][:, None] * aux + betaP[:, t][:, None] * (kt * kt)
            rr = np.log(A) - mu_log[:, None]
            s = rr / (1.0 + np.abs(rr))
            Bv = np.exp(-np.log(x) * s)
            c.update(A=A, rr=rr, B=Bv)
            wt = eta[:, t][:, None] * Bv * kt
            aux = A
        elif gain == "kdn":
            ph = a * a * aux + omega[:, t]
            z = np.sum(ph * kt * kt, axis=1)
            D = r[:, t] + z
            wt = ph * kt / D[:, None]
            u = (mu_info / r[:, t])[:, None] * (kt * kt)
            c.update(ph=ph, D=D, u=u)
            aux = ph / (1.0 + u * ph)
        elif gain == "kdn_iso":
            a2 = np.mean(a * a, axis=1)
            bh = a2 * aux + omega[:, t]
            n = np.sum(kt * kt, axis=1)
            den = r[:, t] + bh * n
            beta = bh / den
            u = mu_info * n / (dk * r[:, t])
            c.update(a2=a2, bh=bh, n=n, den=den, beta=beta, u=u)
            wt = beta[:, None] * kt
            aux = bh / (1.0 + u * bh)
        elif gain == "explicit":
            wt = w_in[:, t]
        else:
            raise ValueError(f"unknown gain {gain!r}")
        e = v[:, t] - np.einsum("nkv,nk->nv", S_dec, kt)
        Sprev.append(S)
        Es.append(e)
        Ws.append(wt)
        cache.append(c)
        S = S_dec + wt[:, :, None] * e[:, None, :]

    # ---- reverse sweep
    g = {n_: np.zeros_like(a_) for n_, a_ in
         (("q", q), ("k", k), ("v", v), ("alpha", alpha)) }
    for name, arr in (("eta", eta), ("alphaP", alphaP), ("betaP", betaP), ("omega", omega),
                      ("r", r), ("w", w_in)):
        if arr is not None:
            g[name] = np.zeros_like(arr)
    if mu_log is not None:
        g["mu_log"] = np.zeros_like(mu_log)
    dS = np.zeros((N, dk, dv)) if dS_T is None else _f64(dS_T).copy()
    daux = None
    if has_aux:
        daux = np.zeros_like(aux) if daux_T is None else _f64(daux_T).reshape(aux.shape).copy()
    for t in range(T - 1, -1, -1):
        kt, qt = k[:, t], q[:, t]
        a = alpha[:, t] if channel else alpha[:, t][:, None]
        S_prev = Sprev[t]
        S_dec = a[:, :, None] * S_prev
        e, wt = Es[t], Ws[t]
        S_t = S_dec + wt[:, :, None] * e[:, None, :]
        # readout o = S_t^T q
        g["q"][:, t] = np.einsum("nkv,nv->nk", S_t, dO[:, t])
        dS = dS + qt[:, :, None] * dO[:, t][:, None, :]
        # write S_t = S_dec + w e^T
        dw = np.einsum("nkv,nv->nk", dS, e)
        de = np.einsum("nkv,nk->nv", dS, wt)
        dS_dec = dS.copy()
        # residual e = v - S_dec^T k
        g["v"][:, t] = de
        g["k"][:, t] -= np.einsum("nkv,nv->nk", S_dec, de)
        dS_dec -= kt[:, :, None] * de[:, None, :]
        # gain
        da_gain, daux = _gain_backward(gain, t, dw, daux, kt, a, channel, cache[t], auxprev[t], g,
                                       eta, eps, alphaP, betaP, mu_log, x, omega, r, mu_info, dk)
        # decay S_dec = a S_{t-1}
        if channel:
            g["alpha"][:, t] += np.einsum("nkv,nkv->nk", dS_dec, S_prev) + da_gain
        else:
            g["alpha"][:, t] += np.einsum("nkv,nkv->n", dS_dec, S_prev) + da_gain.sum(axis=1)
        dS = a[:, :, None] * dS_dec
    g["S0"] = dS
    g["aux0"] = daux
    return g


def _gain_backward(gain, t, dw, daux, kt, a, channel, c, aux_prev, g, eta, eps, alphaP, betaP,
                   mu_log, x, omega, r, mu_info, dk):
    """Back through the write vector w_t = gain(...) and the statistic update.

    dw: dL/dw_t [N, dk]; daux: dL/daux_t (None for gains without one).
    Adds to g["k"][:, t] and the gates' gradients at t; returns
    (da [N, dk] or [N, 1]: the decay's gradient through the gain,
    dL/daux_{t-1}).
    """
    da = np.zeros_like(a)
    if gain == "kla":
        # w = beta k, beta = eta / (n + eps), n = ||k||^2
        n = c["n"]
        beta = eta[:, t] / (n + eps)
        dbeta = np.sum(dw * kt, axis=1)
        g["k"][:, t] += beta[:, None] * dw
        dn = dbeta * (-eta[:, t] / (n + eps) ** 2)
        g["k"][:, t] += 2.0 * dn[:, None] * kt
        g["eta"][:, t] += dbeta / (n + eps)
        return da, None
    if gain == "gdn":
        # w = eta k
        g["k"][:, t] += eta[:, t][:, None] * dw
        g["eta"][:, t] += np.sum(dw * kt, axis=1)
        return da, None
    if gain == "explicit":
        g["w"][:, t] += dw
        return da, None
    if gain == "pgdn":
        # A_t = alphaP A_{t-1} + betaP k^2;  rr = log A_t - mu;  s = rr / (1 + |rr|);
        # B = exp(-log(x) s);  w = eta B k
        A, rr, Bv = c["A"], c["rr"], c["B"]
        et = eta[:, t][:, None]
        g["eta"][:, t] += np.sum(dw * Bv * kt, axis=1)
        g["k"][:, t] += et * Bv * dw
        dB = et * kt * dw
        ds = dB * Bv * (-np.log(x))
        drr = ds / (1.0 + np.abs(rr)) ** 2          # d/drr of rr / (1 + |rr|)
        g["mu_log"] -= np.sum(drr, axis=1)
        dA = drr / A + daux
        g["alphaP"][:, t] += np.sum(dA * aux_prev, axis=1)
        g["betaP"][:, t] += np.sum(dA * kt * kt, axis=1)
        g["k"][:, t] += dA * betaP[:, t][:, None] * 2.0 * kt
        return da, dA * alphaP[:, t][:, None]
    if gain == "kdn":
        # p_hat = a^2 p + omega;  z = sum p_hat k^2;  D = r + z;  w = p_hat k / D;
        # u = (mu / r) k^2;  p_t = p_hat / (1 + u p_hat)
        ph, D, u = c["ph"], c["D"], c["u"]
        rt = r[:, t]
        dph = dw * kt / D[:, None]
        g["k"][:, t] += dw * ph / D[:, None]
        dD = -np.sum(dw * ph * kt, axis=1) / D ** 2
        g["r"][:, t] += dD
        dph += dD[:, None] * kt * kt
        g["k"][:, t] += dD[:, None] * 2.0 * ph * kt
        gg = 1.0 + u * ph
        dph += daux / gg ** 2
        du = -daux * ph * ph / gg ** 2
        g["k"][:, t] += du * (mu_info / rt)[:, None] * 2.0 * kt
        g["r"][:, t] += np.sum(du * kt * kt, axis=1) * (-mu_info / rt ** 2)
        da = dph * 2.0 * a * aux_prev
        g["omega"][:, t] += dph
        return da, dph * a * a
    if gain == "kdn_iso":
        # a2 = mean_i a_i^2;  b_hat = a2 b + omega;  n = ||k||^2;
        # beta = b_hat / (r + b_hat n);  w = beta k;  u = mu n / (d_k r);
        # b_t = b_hat / (1 + u b_hat)
        a2, bh, n, den, beta, u = c["a2"], c["bh"], c["n"], c["den"], c["beta"], c["u"]
        rt = r[:, t]
        dbeta = np.sum(dw * kt, axis=1)
        g["k"][:, t] += beta[:, None] * dw
        dbh = dbeta * rt / den ** 2
        g["r"][:, t] += -dbeta * bh / den ** 2
        dn = -dbeta * bh * bh / den ** 2
        gg = 1.0 + u * bh
        dbh += daux / gg ** 2
        du = -daux * bh * bh / gg ** 2
        dn += du * mu_info / (dk * rt)
        g["r"][:, t] += -du * mu_info * n / (dk * rt ** 2)
        g["k"][:, t] += 2.0 * dn[:, None] * kt
        da2 = dbh * aux_prev
        g["omega"][:, t] += dbh
        da = da2[:, None] * 2.0 * a / a.shape[1]   # a2 = mean over the decay's entries
        return da, dbh * a2
    raise ValueError(f"unknown gain {gain!r}")
