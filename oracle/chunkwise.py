"""The chunkwise (triangular-system) form of the recurrence in fp64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The same chunk equations as oracle.exact.chunkwise (Kaczmarz Linear
Attention §2.5 Eqs. 7-9; Preconditioned DeltaNet §2.6 Eq. 6; extended to
per-channel decay), with numpy products and a plain forward substitution,
for all gains including pgdn.  Cumulative decay is formed from log-decay
sums (Kalman Delta Networks §2.6 numerics: decay ratios from differences of
cumulative log-decay).  The write vectors come from
oracle.recurrence.forward's trace; this module checks the state/readout
part of the chunk form at any size, where exact rationals are too slow.
"""
from __future__ import annotations

import numpy as np


def forward(q, k, v, w, alpha, C, S0=None):
    """q, k, w [N, T, dk]; v [N, T, dv]; alpha [N, T] or [N, T, dk].

    Returns (o [N, T, dv], S_T [N, dk, dv]).
    """
    q, k, v, w, alpha = (np.asarray(a, np.float64) for a in (q, k, v, w, alpha))
    N, T, dk = k.shape
    dv = v.shape[-1]
    if alpha.ndim == 2:
        alpha = np.repeat(alpha[:, :, None], dk, axis=2)
    S = np.zeros((N, dk, dv)) if S0 is None else np.asarray(S0, np.float64).copy()
    o = np.zeros((N, T, dv))
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        sl = slice(c0, c0 + n)
        G = np.cumsum(np.log(alpha[:, sl]), axis=1)  # [N, n, dk]
        g = np.exp(G)
        Kh, Qh = g * k[:, sl], g * q[:, sl]
        Wc = w[:, sl] * np.exp(-G)
        Wt = w[:, sl] * np.exp(G[:, -1:, :] - G)
        L = np.tril(np.einsum("nid,njd->nij", Kh, Wc), -1)
        M = np.tril(np.einsum("nid,njd->nij", Qh, Wc), 0)
        R = v[:, sl] - np.einsum("nid,ndj->nij", Kh, S)
        U = np.zeros_like(R)
        for i in range(n):
            U[:, i] = R[:, i] - np.einsum("nm,nmj->nj", L[:, i, :i], U[:, :i])
        o[:, sl] = np.einsum("nid,ndj->nij", Qh, S) + np.einsum("nim,nmj->nij", M, U)
        S = g[:, -1, :, None] * S + np.einsum("nmd,nmj->ndj", Wt, U)
    return o, S
