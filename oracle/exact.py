"""The recurrence and its chunkwise form in exact rational arithmetic.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Tiny single-head inputs as Python lists of fractions.Fraction.  Gains whose
arithmetic stays rational are supported: kla, gdn, kdn and explicit (pgdn
takes log/exp and is pinned in fp64 instead); kdn_iso as well, with
scalar omega_t and the variance b as a one-element list.

token_recurrence follows the same five steps as oracle.recurrence.forward
(Kaczmarz Linear Attention §2.1; Kalman Delta Networks §1.1 and §2.4-2.5).

chunkwise evaluates the chunk form, our single statement of Kaczmarz Linear
Attention §2.5 (Eqs. 7-9) and Preconditioned DeltaNet §2.6 (Eq. 6),
extended to per-channel decay.  For a chunk of n tokens with input state
S_in and cumulative decay g_i = prod_{r<=i} alpha_r (per channel):

    khat_i = g_i * k_i,   qhat_i = g_i * q_i,   wchk_j = w_j / g_j,
    wtil_j = (g_n / g_j) * w_j
    L_ij = khat_i . wchk_j  (j < i),   M_ij = qhat_i . wchk_j  (j <= i)
    (I + L) U = V - Khat S_in           (unit lower-triangular; row i of U
                                         is the residual e_i of token i)
    O = Qhat S_in + M U,   S_out = diag(g_n) S_in + Wtil^T U

Exact equality with token_recurrence on every input is the pin that the
chunk equations reach the recurrence, not an approximation of it.
"""
from __future__ import annotations

from fractions import Fraction as F
from typing import List, Optional, Sequence

Vec = List[F]
Mat = List[List[F]]


def _dot(a: Sequence[F], b: Sequence[F]) -> F:
    return sum((x * y for x, y in zip(a, b)), F(0))


def _zeros(r: int, c: int) -> Mat:
    return [[F(0)] * c for _ in range(r)]


def gains(k: Mat, gain: str, alpha, eta=None, eps=F(0), omega=None, r=None,
          mu_info=F(1), w=None, p0: Optional[Vec] = None):
    """Per-token write vectors w_t (and the KDN variance after each token)."""
    T, dk = len(k), len(k[0])
    ws, ps = [], []
    p = list(p0) if p0 is not None else [F(1)] * (1 if gain == "kdn_iso" else dk)
    for t in range(T):
        kt = k[t]
        a = alpha[t] if isinstance(alpha[t], list) else [alpha[t]] * dk
        if gain == "kla":
            beta = eta[t] / (_dot(kt, kt) + eps)
            ws.append([beta * x for x in kt])
        elif gain == "gdn":
            ws.append([eta[t] * x for x in kt])
        elif gain == "kdn":
            p_hat = [a[i] * a[i] * p[i] + omega[t][i] for i in range(dk)]
            z = sum((p_hat[i] * kt[i] * kt[i] for i in range(dk)), F(0))
            ws.append([p_hat[i] * kt[i] / (r[t] + z) for i in range(dk)])
            u = [mu_info / r[t] * kt[i] * kt[i] for i in range(dk)]
            p = [p_hat[i] / (1 + u[i] * p_hat[i]) for i in range(dk)]
            ps.append(list(p))
        elif gain == "kdn_iso":
            # Kalman Delta Networks §2.7, Eq. 40 (p holds the one variance b)
            b_hat = sum((x * x for x in a), F(0)) / dk * p[0] + omega[t]
            n = _dot(kt, kt)
            beta = b_hat / (r[t] + b_hat * n)
            ws.append([beta * x for x in kt])
            u = mu_info * n / (dk * r[t])
            p = [b_hat / (1 + u * b_hat)]
            ps.append(list(p))
        elif gain == "explicit":
            ws.append(list(w[t]))
        else:
            raise ValueError(f"gain {gain!r} is not rational")
    return ws, ps


def token_recurrence(q: Mat, k: Mat, v: Mat, ws: Mat, alpha, S0: Optional[Mat] = None):
    """o_t and S_T of the recurrence with given write vectors w_t."""
    T, dk, dv = len(k), len(k[0]), len(v[0])
    S = [row[:] for row in S0] if S0 is not None else _zeros(dk, dv)
    o = []
    for t in range(T):
        a = alpha[t] if isinstance(alpha[t], list) else [alpha[t]] * dk
        S_dec = [[a[i] * S[i][j] for j in range(dv)] for i in range(dk)]
        e = [v[t][j] - sum((S_dec[i][j] * k[t][i] for i in range(dk)), F(0)) for j in range(dv)]
        S = [[S_dec[i][j] + ws[t][i] * e[j] for j in range(dv)] for i in range(dk)]
        o.append([sum((S[i][j] * q[t][i] for i in range(dk)), F(0)) for j in range(dv)])
    return o, S


def chunkwise(q: Mat, k: Mat, v: Mat, ws: Mat, alpha, C: int, S0: Optional[Mat] = None):
    """o_t and S_T via the chunk form (forward substitution per chunk)."""
    T, dk, dv = len(k), len(k[0]), len(v[0])
    S = [row[:] for row in S0] if S0 is not None else _zeros(dk, dv)
    o: Mat = []
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        # cumulative decay per channel
        g: Mat = []
        run = [F(1)] * dk
        for i in range(n):
            a = alpha[c0 + i] if isinstance(alpha[c0 + i], list) else [alpha[c0 + i]] * dk
            run = [run[d] * a[d] for d in range(dk)]
            g.append(run)
        K = [[g[i][d] * k[c0 + i][d] for d in range(dk)] for i in range(n)]
        Qh = [[g[i][d] * q[c0 + i][d] for d in range(dk)] for i in range(n)]
        Wc = [[ws[c0 + j][d] / g[j][d] for d in range(dk)] for j in range(n)]
        Wt = [[g[n - 1][d] / g[j][d] * ws[c0 + j][d] for d in range(dk)] for j in range(n)]
        L = [[_dot(K[i], Wc[j]) if j < i else F(0) for j in range(n)] for i in range(n)]
        M = [[_dot(Qh[i], Wc[j]) if j <= i else F(0) for j in range(n)] for i in range(n)]
        # right-hand side V - Khat S_in, then forward substitution
        R = [[v[c0 + i][j] - sum((K[i][d] * S[d][j] for d in range(dk)), F(0))
              for j in range(dv)] for i in range(n)]
        U: Mat = []
        for i in range(n):
            U.append([R[i][j] - sum((L[i][m] * U[m][j] for m in range(i)), F(0))
                      for j in range(dv)])
        for i in range(n):
            o.append([sum((Qh[i][d] * S[d][j] for d in range(dk)), F(0))
                      + sum((M[i][m] * U[m][j] for m in range(i + 1)), F(0))
                      for j in range(dv)])
        S = [[g[n - 1][d] * S[d][j] + sum((Wt[m][d] * U[m][j] for m in range(n)), F(0))
              for j in range(dv)] for d in range(dk)]
    return o, S
