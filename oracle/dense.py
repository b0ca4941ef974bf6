"""Dense-covariance Kalman associative memory in fp64 (numpy).

TEST INFRASTRUCTURE ONLY: a brute-force reference used by the CPU tests to
pin the KDN oracle.  It is never imported by the GPU library.

It follows the belief-state recursion of the Bayesian Layer ("Memory by
Design: Probabilistic Sequence Layers", section 2.2, Proposition 1), which
is the exact Kalman filter for a matrix memory whose columns share one dense
key-space covariance:

    P_bar = A P A^T + Q                 predicted covariance
    u     = P_bar k                     uncertainty-warped key
    beta  = 1 / (R + k^T u)             innovation precision
    M     = (I - beta u k^T) A M + beta u v^T      mean update
    P     = P_bar - beta u u^T          covariance update
    y     = M^T q                       readout

Symbols are mapped to the KDN pages ("Kalman Delta Networks", section 3):
R is the observation-noise variance (r_t on the KDN pages, r^2 on the
Bayesian Layer page), Q the process-noise covariance (diag(omega_t) on the
KDN pages, l^2 I on the Bayesian Layer page) and A the transition
(diag(alpha_t) on the KDN pages).  The gate form written here is a different
expression of the same update than the residual write the KDN oracle uses,
which is what makes the two useful against each other.
"""
from __future__ import annotations

import numpy as np


def dense_step(M, P, k, v, A, Q, R, q=None, P_bar_override=None):
    """One predict/update step of the dense filter.

    M [D,m], P [D,D], k [D], v [m], A [D,D], Q [D,D], R scalar, q [D] or None.
    ``P_bar_override`` replaces the predicted covariance (the covariance-reset
    ablation of the Bayesian Layer page, appendix E.4.1).
    Returns (M_new, P_new, y, u, beta) with y = M_new^T q (None if q is None).
    """
    M = np.asarray(M, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    P_bar = A @ P @ A.T + Q if P_bar_override is None else np.asarray(P_bar_override, np.float64)
    u = P_bar @ k
    beta = 1.0 / (R + k @ u)
    D = len(k)
    gate = np.eye(D) - beta * np.outer(u, k)
    M_new = gate @ (A @ M) + beta * np.outer(u, v)
    P_new = P_bar - beta * np.outer(u, u)
    y = None if q is None else M_new.T @ np.asarray(q, np.float64)
    return M_new, P_new, y, u, beta


def dense_filter(keys, values, A_seq, Q_seq, R_seq, P0, M0=None, queries=None):
    """Run dense_step over a sequence.

    keys [T,D], values [T,m], A_seq [T,D,D], Q_seq [T,D,D], R_seq [T],
    P0 [D,D]; queries [T,D] or None.  Returns dict with per-step M, P, y, u, beta.
    """
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    T, D = keys.shape
    m = values.shape[1]
    M = np.zeros((D, m)) if M0 is None else np.array(M0, np.float64)
    P = np.array(P0, np.float64)
    out = {"M": [], "P": [], "y": [], "u": [], "beta": []}
    for t in range(T):
        q = None if queries is None else queries[t]
        M, P, y, u, beta = dense_step(M, P, keys[t], values[t], A_seq[t], Q_seq[t], R_seq[t], q)
        out["M"].append(M)
        out["P"].append(P)
        out["y"].append(y)
        out["u"].append(u)
        out["beta"].append(beta)
    return out
