"""Second float64 transcription of the CKDA recurrence, in numpy -- TEST
INFRASTRUCTURE ONLY (tiny shapes; pure Python loop over tokens).

It restates the same definition as ``ckda_oracle.c`` in matrix notation so
that a transcription slip in either one shows up as a disagreement:

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t,       alpha_t = s_t * exp(g_t)

(Complex KDA paper page, sections 2-3: the DeltaNet transition with KDA's
channel-wise gate, gate range [-1, 1], beta range [0, 2].)  The transition
matrix is built explicitly here, whereas the C code never forms it.
"""
from __future__ import annotations

import numpy as np


def transition(k: np.ndarray, alpha: np.ndarray, beta: float) -> np.ndarray:
    """A = (I - beta k k^T) Diag(alpha), a DK x DK matrix."""
    d = k.shape[0]
    return (np.eye(d) - beta * np.outer(k, k)) @ np.diag(alpha)


def fwd_chain(q, k, v, g, s, beta, scale=1.0, S0=None):
    """One chain: q,k,g,s [T,DK], v [T,DV], beta [T].  Returns (o [T,DV], S_T)."""
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, DV))
    for t in range(T):
        alpha = s[t] * np.exp(g[t])
        S = transition(k[t], alpha, beta[t]) @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = scale * (S.T @ q[t])
    return o, S


def bwd_chain(q, k, v, g, s, beta, do, scale=1.0, S0=None, dST=None):
    """Reverse mode of L = sum_t <do_t, o_t> + <dST, S_T> using the explicit
    transition matrices.  Returns dict dq, dk, dv, dg, dbeta, dS0."""
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    states = [S]
    for t in range(T):
        alpha = s[t] * np.exp(g[t])
        S = transition(k[t], alpha, beta[t]) @ S + beta[t] * np.outer(k[t], v[t])
        states.append(S)
    dS = np.zeros((DK, DV)) if dST is None else np.array(dST, dtype=np.float64)
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g))}
    out["dbeta"] = np.zeros(T)
    I = np.eye(DK)
    for t in range(T - 1, -1, -1):
        Sp, St = states[t], states[t + 1]
        alpha = s[t] * np.exp(g[t])
        D = np.diag(alpha)
        kt, bt = k[t], beta[t]
        # o_t = scale * S_t^T q_t
        out["dq"][t] = scale * (St @ do[t])
        dS = dS + scale * np.outer(q[t], do[t])
        # S_t = (I - b k k^T) D Sp + b k v^T
        X = D @ Sp                                   # gated previous state
        dX = (I - bt * np.outer(kt, kt)).T @ dS      # dL/d(D Sp)
        # d/dk of -b k k^T X  and  b k v^T
        kX = kt @ X                                  # k^T X   [DV]
        out["dk"][t] = -bt * (dS @ kX + X @ (dS.T @ kt)) + bt * dS @ v[t]
        out["dbeta"][t] = -np.sum(dS * np.outer(kt, kX)) + np.sum(dS * np.outer(kt, v[t]))
        out["dv"][t] = bt * (dS.T @ kt)
        # X = Diag(alpha) Sp, alpha = s e^g  ->  dL/dg = alpha * rowsum(dX * Sp)
        out["dg"][t] = alpha * np.sum(dX * Sp, axis=1)
        dS = D @ dX
    out["dS0"] = dS
    return out
