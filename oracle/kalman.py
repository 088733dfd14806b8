"""Textbook estimators used as independent pins of the recurrence.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

dense_kalman   The exact Kalman filter of the linear-Gaussian memory model
               with a dense key-space covariance shared by all value columns
               (Kalman Delta Networks §2.1-2.2, Eqs. 12-17): predict
               S_hat = D S, P_hat = D P D^T + Omega; gain
               kappa = P_hat k / (r + k^T P_hat k); update
               S = S_hat + kappa (v - S_hat^T k)^T, P = (I - kappa k^T) P_hat.

ridge          Ridge regression S* = (lambda I + K^T K)^{-1} K^T V, in this
               build's d_k x d_v orientation (Preconditioned DeltaNet §2.1,
               Eqs. 1-2), solved by numpy.linalg.solve.

atk_write_vectors
               The exact apply-to-key write vectors
               w_t = P_{t-1} k_t / (1 + k_t^T P_{t-1} k_t) with the
               Sherman-Morrison inverse-Gram update, P_0 = I / lambda
               (Preconditioned DeltaNet §2.2, Eqs. 3-5).
"""
from __future__ import annotations

import numpy as np


def dense_kalman(k, v, D, Omega, r, S0, P0):
    """k [T, dk], v [T, dv], D and Omega [T, dk, dk], r [T]; returns S_T, P_T, kappas."""
    S, P = np.array(S0, np.float64), np.array(P0, np.float64)
    kappas = []
    for t in range(len(k)):
        Dt = D[t]
        S_hat = Dt @ S
        P_hat = Dt @ P @ Dt.T + Omega[t]
        kt = k[t]
        kappa = P_hat @ kt / (r[t] + kt @ P_hat @ kt)
        S = S_hat + np.outer(kappa, v[t] - S_hat.T @ kt)
        P = (np.eye(len(kt)) - np.outer(kappa, kt)) @ P_hat
        kappas.append(kappa)
    return S, P, np.array(kappas)


def ridge(K, V, lam):
    dk = K.shape[1]
    return np.linalg.solve(lam * np.eye(dk) + K.T @ K, K.T @ V)


def atk_write_vectors(K, lam):
    """Write vectors of exact ATK and the final inverse Gram P_T."""
    dk = K.shape[1]
    P = np.eye(dk) / lam
    ws = []
    for kt in K:
        Pk = P @ kt
        denom = 1.0 + kt @ Pk
        ws.append(Pk / denom)
        P = P - np.outer(Pk, Pk) / denom
    return np.array(ws), P
