"""Chunked (UT/WY) form of the CKDA recurrence in float64 numpy -- test helper.

This is NOT the oracle: it restates, in plain numpy, the chunk-wise algebra the
GPU kernels implement, so a test can show that the algebra reproduces the token
recurrence (up to float64 rounding) independently of any kernel.  Notation per
chunk of L <= 64 tokens, in the chunk-local folded frame (the sign product P
restarts at +1 at every chunk; the "complex-kda-1.3B-100B" model card describes
pushing the running sign product onto q and k):

  b_r   = sum_{i<=r} g_i                  (per channel; g = log|alpha|)
  P_r   = prod_{i<=r} s_i                 q~ = P*q,  k~ = P*k
  A_ri  = sum_c k~_rc k~_ic e^{b_rc-b_ic}  (i < r)   M_ri = same with q~_r, i <= r
  X     = I + Diag(beta) A               (unit lower triangular)
  U     = X^{-1} Diag(beta) (V - (k~ e^b) S)          S = state at chunk start
  O     = (q~ e^b) S + M U
  S'    = Diag(P_L e^{b_L}) S + Diag(P_L) (k~ e^{b_L - b})^T U

The paper page (section 2, "Linear RNNs") credits KDA-type models with WY-based
chunk-wise implementations; this is that form for the signed gate.
Optionally the exponentials of the intra-chunk products are anchored per
16-row block the way the kernels do it (``anchored=True``).
"""
from __future__ import annotations

import numpy as np


def _intra(qt, kt, b, anchored: bool, blk: int = 16):
    L, DK = kt.shape
    if not anchored:
        E = np.exp(b)
        Ei = np.exp(-b)
        A = (kt * E) @ (kt * Ei).T
        M = (qt * E) @ (kt * Ei).T
    else:
        A = np.zeros((L, L))
        M = np.zeros((L, L))
        nb = (L + blk - 1) // blk
        for I in range(nb):
            i0, i1 = I * blk, min(L, I * blk + blk)
            m = b[min(i0 + blk // 2 - 1, i1 - 1)]          # anchor: middle row of column block I
            col = kt[i0:i1] * np.exp(m - b[i0:i1])
            rows = slice(i0, L)
            rk = kt[rows] * np.exp(b[rows] - m)
            rq = qt[rows] * np.exp(b[rows] - m)
            A[rows, i0:i1] = rk @ col.T
            M[rows, i0:i1] = rq @ col.T
    A = np.tril(A, -1)
    M = np.tril(M, 0)
    return A, M


def fwd_chain(q, k, v, g, s, beta, scale=1.0, S0=None, C=64, anchored=True):
    """One chain.  q,k,g,s: [T,DK]; v: [T,DV]; beta: [T].  Returns (o, S_T)."""
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, DV))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        L = c1 - c0
        b = np.cumsum(g[c0:c1], axis=0)
        P = np.cumprod(s[c0:c1], axis=0)
        qt = P * q[c0:c1]
        kt = P * k[c0:c1]
        A, M = _intra(qt, kt, b, anchored)
        bt = beta[c0:c1]
        X = np.eye(L) + bt[:, None] * A
        Rm = v[c0:c1] - (kt * np.exp(b)) @ S
        U = np.linalg.solve(X, bt[:, None] * Rm)
        o[c0:c1] = scale * ((qt * np.exp(b)) @ S + M @ U)
        bL, PL = b[-1], P[-1]
        kbar = kt * np.exp(bL - b)
        S = (PL * np.exp(bL))[:, None] * S + PL[:, None] * (kbar.T @ U)
    return o, S


def chunk_record(q, k, v, g, s, beta, C=64):
    """The per-chunk record of the two-kernel forward, for one chunk (L <= C
    tokens): everything that does not depend on the state.
        W = T (kf e^b),  u = T V,  Qh = qf e^b,  KbT = (P_L kf e^{b_L - b})^T,
        M (lower),  d = P_L e^{b_L},   T = (I + Diag(beta) A)^{-1} Diag(beta)"""
    b = np.cumsum(g, axis=0)
    P = np.cumprod(s, axis=0)
    qt, kt = P * q, P * k
    A, M = _intra(qt, kt, b, anchored=True)
    L = q.shape[0]
    Tm = np.linalg.solve(np.eye(L) + beta[:, None] * A, np.diag(beta))
    return dict(W=Tm @ (kt * np.exp(b)), u=Tm @ v, Qh=qt * np.exp(b),
                KbT=(P[-1] * kt * np.exp(b[-1] - b)).T, M=M, d=P[-1] * np.exp(b[-1]))


def fwd_chain_record(q, k, v, g, s, beta, scale=1.0, S0=None, C=64):
    """The state pass over chunk records: U = u - W S, O = scale (Qh S + M U),
    S <- Diag(d) S + KbT U.  Returns (o, S_T)."""
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, DV))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        r = chunk_record(q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], s[c0:c1], beta[c0:c1], C)
        U = r["u"] - r["W"] @ S
        o[c0:c1] = scale * (r["Qh"] @ S + r["M"] @ U)
        S = r["d"][:, None] * S + r["KbT"] @ U
    return o, S


def bwd_chain(q, k, v, g, s, beta, do, scale=1.0, S0=None, dST=None, C=64):
    """Chunk-wise reverse mode of L = <do, o> + <dST, S_T>, same notation as
    fwd_chain (unanchored exponentials; float64 only).  Returns dict dq, dk,
    dv, dg, dbeta, dS0."""
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    starts = list(range(0, T, C))
    hs = []
    for c0 in starts:                              # forward: chunk-start states
        hs.append(S.copy())
        c1 = min(T, c0 + C)
        _, S = fwd_chain(q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], s[c0:c1], beta[c0:c1],
                         scale, S, C=C, anchored=False)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros_like(g), dbeta=np.zeros_like(beta))
    dS = np.zeros((DK, DV)) if dST is None else np.array(dST, dtype=np.float64)
    for ci in range(len(starts) - 1, -1, -1):
        c0 = starts[ci]
        c1 = min(T, c0 + C)
        L = c1 - c0
        S = hs[ci]
        b = np.cumsum(g[c0:c1], axis=0)
        P = np.cumprod(s[c0:c1], axis=0)
        qt, kt = P * q[c0:c1], P * k[c0:c1]
        G = np.exp(b)
        bL, PL = b[-1], P[-1]
        GL = np.exp(bL)
        qh, kh, kc = qt * G, kt * G, kt / G
        kbar = kt * (GL / G)
        A = np.tril(kh @ kc.T, -1)
        M = np.tril(qh @ kc.T, 0)
        bt = beta[c0:c1]
        V = v[c0:c1]
        X = np.eye(L) + bt[:, None] * A
        Xi = np.linalg.inv(X)
        Tm = Xi * bt[None, :]
        W = Tm @ kh
        U = Tm @ V - W @ S
        dO = scale * do[c0:c1]
        dSt = PL[:, None] * dS                      # gradient w.r.t. folded chunk-end state
        dU = M.T @ dO + kbar @ dSt
        dM = np.tril(dO @ U.T, 0)
        dS_prev = qh.T @ dO + GL[:, None] * dSt - W.T @ dU
        dkbar = U @ dSt.T
        dGL = np.sum(dSt * S, axis=1)
        dW = -dU @ S.T
        dV = Tm.T @ dU
        dT = dU @ V.T + dW @ kh.T
        dkh = Tm.T @ dW
        dXi = dT * bt[None, :]
        dbeta = np.sum(dT * Xi, axis=0)
        dX = -Xi.T @ dXi @ Xi.T
        dXs = np.tril(dX, -1)
        dbeta += np.sum(dXs * A, axis=1)
        dA = bt[:, None] * dXs
        dkh += dA @ kc
        dkc = dA.T @ kh + dM.T @ qh
        dqh = dM @ kc + dO @ S.T
        dqt = dqh * G
        dkt = dkh * G + dkc / G + dkbar * (GL / G)
        db = qh * dqh + kh * dkh - kc * dkc - kbar * dkbar
        db[-1] += np.sum(kbar * dkbar, axis=0) + GL * dGL
        dg = np.cumsum(db[::-1], axis=0)[::-1]
        out["dq"][c0:c1] = P * dqt
        out["dk"][c0:c1] = P * dkt
        out["dv"][c0:c1] = dV
        out["dg"][c0:c1] = dg
        out["dbeta"][c0:c1] = dbeta
        dS = dS_prev
    out["dS0"] = dS
    return out


def bwd_chain_anchored(q, k, v, g, s, beta, do, scale=1.0, S0=None, dST=None, C=64):
    """The same reverse mode written in the anchored variables the GPU
    backward uses: with m = b at the chunk's token 31,
        K1 = kf e^{b-m},  K2 = kf e^{m-b},  Q1 = qf e^{b-m},  KB = kf e^{b_L-b},
        S' = Diag(e^m) S.
    e^{b_r - b_i} = (K1 K2^T)_ri / (kf kf) etc.; every factor stays within the
    span of half a chunk, and the gate gradient db keeps its form because
    the anchors cancel."""
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    starts = list(range(0, T, C))
    hs = []
    for c0 in starts:
        hs.append(S.copy())
        c1 = min(T, c0 + C)
        _, S = fwd_chain(q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], s[c0:c1], beta[c0:c1],
                         scale, S, C=C, anchored=False)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros_like(g), dbeta=np.zeros_like(beta))
    G = np.zeros((DK, DV)) if dST is None else np.array(dST, dtype=np.float64)
    for ci in range(len(starts) - 1, -1, -1):
        c0 = starts[ci]
        c1 = min(T, c0 + C)
        L = c1 - c0
        S = hs[ci]
        b = np.cumsum(g[c0:c1], axis=0)
        P = np.cumprod(s[c0:c1], axis=0)
        qt, kt = P * q[c0:c1], P * k[c0:c1]
        m = b[min(31, L - 1)]
        bL, PL = b[-1], P[-1]
        K1, K2, Q1 = kt * np.exp(b - m), kt * np.exp(m - b), qt * np.exp(b - m)
        KB = kt * np.exp(bL - b)
        Sp = np.exp(m)[:, None] * S
        A = np.tril(K1 @ K2.T, -1)
        M = np.tril(Q1 @ K2.T, 0)
        bt = beta[c0:c1]
        V = v[c0:c1]
        Xi = np.linalg.inv(np.eye(L) + bt[:, None] * A)
        Tm = Xi * bt[None, :]
        U = Tm @ (V - K1 @ Sp)
        dO = scale * do[c0:c1]
        dSt = PL[:, None] * G
        dU = M.T @ dO + KB @ dSt
        Z = Tm.T @ dU
        G = np.exp(m)[:, None] * (Q1.T @ dO - K1.T @ Z) + np.exp(bL)[:, None] * dSt
        dM = np.tril(dO @ U.T, 0)
        dKB = U @ dSt.T
        dGL = np.sum(dSt * S, axis=1)
        dWp = -dU @ Sp.T
        dV = Tm.T @ dU
        dT = dU @ V.T + dWp @ K1.T
        dK1 = Tm.T @ dWp
        dbeta = np.sum(dT * Xi, axis=0)
        dX = -Xi.T @ (dT * bt[None, :]) @ Xi.T
        dXs = np.tril(dX, -1)
        dbeta += np.sum(dXs * A, axis=1)
        dA = bt[:, None] * dXs
        dK1 += dA @ K2
        dK2 = dA.T @ K1 + dM.T @ Q1
        dQ1 = dM @ K2 + dO @ Sp.T
        dqt = dQ1 * np.exp(b - m)
        dkt = dK1 * np.exp(b - m) + dK2 * np.exp(m - b) + dKB * np.exp(bL - b)
        db = Q1 * dQ1 + K1 * dK1 - K2 * dK2 - KB * dKB
        db[-1] += np.sum(KB * dKB, axis=0) + np.exp(bL) * dGL
        out["dq"][c0:c1] = P * dqt
        out["dk"][c0:c1] = P * dkt
        out["dv"][c0:c1] = dV
        out["dg"][c0:c1] = np.cumsum(db[::-1], axis=0)[::-1]
        out["dbeta"][c0:c1] = dbeta
    out["dS0"] = G
    return out
