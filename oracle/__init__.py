"""CPU oracle for the Complex KDA (CKDA) recurrence -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library (``libckda.so``) and
its binding never import, link or call anything here, and share no code with
it.

``ckda_oracle.c`` holds the plain float64 token-by-token recurrence (forward,
folded-frame forward, backward); this module lays the caller's tensors out as
independent chains (one per sequence or document and head) and calls it
through ctypes.  ``ref_numpy`` is a second, independent float64 transcription
in numpy used to cross-check the C code on tiny shapes.

Tensor conventions (all float64 on the way in and out):
  q, k, g, s: [B, T, H, DK]   v, o, do: [B, T, H, DV]   beta: [B, T, H]
  states:     [B, H, DK, DV]  (row = key channel, column = value channel)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ckda_oracle.c")
_LIB = os.path.join(_HERE, "libckda_oracle.so")
_lib = None

BUILD_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
             "-o", _LIB, _SRC, "-lm"]


def build(force: bool = True) -> str:
    """Compile the C oracle into oracle/libckda_oracle.so."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = list(BUILD_CMD)
        cmd[cmd.index(_LIB)] = tmp
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("CKDA_ORACLE_LIB")   # another build of the same source (sanitizer runs)
        if not path:
            if not os.path.exists(_LIB):
                build(force=True)
            path = _LIB
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.ckda_ref_fwd.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, ctypes.c_double,
                                     dp, dp, dp]
        lib.ckda_ref_fwd.restype = i
        lib.ckda_ref_fwd_folded.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp,
                                            ctypes.c_double, dp, dp, dp, dp, dp]
        lib.ckda_ref_fwd_folded.restype = i
        lib.ckda_ref_bwd.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, ctypes.c_double,
                                     dp, dp, dp, i, dp, dp, dp, dp, dp, dp]
        lib.ckda_ref_bwd.restype = i
        lib.ckda_ref_set_threads.argtypes = [i]
        lib.ckda_ref_max_threads.restype = i
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    _load().ckda_ref_set_threads(int(n))


def max_threads() -> int:
    return int(_load().ckda_ref_max_threads())


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _chains(x: np.ndarray) -> np.ndarray:
    """[B, T, H, D] -> contiguous [B*H, T, D] float64."""
    B, T, H, D = x.shape
    return np.ascontiguousarray(np.asarray(x, np.float64).transpose(0, 2, 1, 3).reshape(B * H, T, D))


def _unchain(x: np.ndarray, B: int, H: int) -> np.ndarray:
    n, T, D = x.shape
    return x.reshape(B, H, T, D).transpose(0, 2, 1, 3)


# ----------------------------------------------------------------------------
# chain-level entry points (n independent chains, each contiguous)
# ----------------------------------------------------------------------------
def fwd_chain_arrays(q, k, v, g, s, beta, scale=1.0, S0=None):
    """q,k,g,s: [n,T,DK]; v: [n,T,DV]; beta: [n,T]; S0: [n,DK,DV] or None."""
    q, k, v, g, s, beta = (np.ascontiguousarray(a, np.float64) for a in (q, k, v, g, s, beta))
    n, T, DK = q.shape
    DV = v.shape[2]
    o = np.empty((n, T, DV))
    ST = np.empty((n, DK, DV))
    S0c = None if S0 is None else np.ascontiguousarray(S0, np.float64)
    rc = _load().ckda_ref_fwd(n, T, DK, DV, _p(q), _p(k), _p(v), _p(g), _p(s), _p(beta),
                              float(scale), _p(S0c), _p(o), _p(ST))
    if rc != 0:
        raise RuntimeError(f"ckda_ref_fwd failed ({rc})")
    return o, ST


def fwd_folded_chain_arrays(q, k, v, g, s, beta, scale=1.0, S0=None, P0=None):
    q, k, v, g, s, beta = (np.ascontiguousarray(a, np.float64) for a in (q, k, v, g, s, beta))
    n, T, DK = q.shape
    DV = v.shape[2]
    o = np.empty((n, T, DV))
    ST = np.empty((n, DK, DV))
    PT = np.empty((n, DK))
    S0c = None if S0 is None else np.ascontiguousarray(S0, np.float64)
    P0c = None if P0 is None else np.ascontiguousarray(P0, np.float64)
    rc = _load().ckda_ref_fwd_folded(n, T, DK, DV, _p(q), _p(k), _p(v), _p(g), _p(s), _p(beta),
                                     float(scale), _p(S0c), _p(P0c), _p(o), _p(ST), _p(PT))
    if rc != 0:
        raise RuntimeError(f"ckda_ref_fwd_folded failed ({rc})")
    return o, ST, PT


def bwd_chain_arrays(q, k, v, g, s, beta, do, scale=1.0, S0=None, dST=None, every=64):
    q, k, v, g, s, beta, do = (np.ascontiguousarray(a, np.float64)
                               for a in (q, k, v, g, s, beta, do))
    n, T, DK = q.shape
    DV = v.shape[2]
    dq = np.empty((n, T, DK)); dk = np.empty((n, T, DK)); dg = np.empty((n, T, DK))
    dv = np.empty((n, T, DV)); dbeta = np.empty((n, T)); dS0 = np.empty((n, DK, DV))
    S0c = None if S0 is None else np.ascontiguousarray(S0, np.float64)
    dSTc = None if dST is None else np.ascontiguousarray(dST, np.float64)
    rc = _load().ckda_ref_bwd(n, T, DK, DV, _p(q), _p(k), _p(v), _p(g), _p(s), _p(beta),
                              float(scale), _p(S0c), _p(do), _p(dSTc), int(every),
                              _p(dq), _p(dk), _p(dv), _p(dg), _p(dbeta), _p(dS0))
    if rc != 0:
        raise RuntimeError(f"ckda_ref_bwd failed ({rc})")
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dS0=dS0)


# ----------------------------------------------------------------------------
# per-head L2 normalisation of q and k (the unit keys of the Complex KDA paper
# page, sections 3-4), written out: y = x / ||x|| over the key channels, with
# a zero vector left at zero; its reverse mode dx = (dy - y (y . dy)) / ||x||.
# ----------------------------------------------------------------------------
def l2norm(x) -> np.ndarray:
    x = np.asarray(x, np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def l2norm_bwd(x, dy) -> np.ndarray:
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    y = np.divide(x, n, out=np.zeros_like(x), where=n > 0)
    r = dy - y * np.sum(y * dy, axis=-1, keepdims=True)
    return np.divide(r, n, out=np.zeros_like(x), where=n > 0)


# ----------------------------------------------------------------------------
# Optional gate map (the CKDA_GATE_MAP option).  The Complex KDA paper page,
# section 3, paragraph "CKDA.", defines CKDA as KDA with gates in [-1, 1] and
# the delta-rule coefficient beta in [0, 2], built with a signed gate and a
# beta range extension after Sarrof et al. (2024) and Grazzi et al. (2025),
# "with the magnitude floor and backward convention" of an appendix the pages
# do not include; the formulas themselves did not survive.  Reading taken
# here (parity unpinned for the floor and the gate's functional form):
#   alpha = tanh(x)               (a signed gate in (-1, 1))
#   s     = -1 if x < 0 else +1   (x = 0 counts as +1)
#   g     = log max(|alpha|, e^GATE_LOG_FLOOR)   (the magnitude floor)
#   beta  = 2 sigmoid(y)          (beta in (0, 2))
# and the backward is the plain derivative: dg/dx = (1 - tanh^2 x) / tanh x
# above the floor, 0 on it; s gets no gradient; dbeta/dy = beta (1 - beta/2).
# ----------------------------------------------------------------------------
GATE_LOG_FLOOR = -4.0


def gate_map(x, y):
    """(g, s, beta) from the gate pre-activation x and beta pre-activation y."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    t = np.abs(np.tanh(x))
    with np.errstate(divide="ignore"):
        g = np.maximum(np.log(t), GATE_LOG_FLOOR)
    s = np.where(x < 0, -1.0, 1.0)
    beta = 2.0 / (1.0 + np.exp(-y))
    return g, s, beta


def gate_map_bwd(x, y, dg, dbeta):
    """(dL/dx, dL/dy) from dL/dg and dL/dbeta through gate_map."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    th = np.tanh(x)
    above = np.abs(th) >= np.exp(GATE_LOG_FLOOR)
    with np.errstate(divide="ignore", invalid="ignore"):
        dgdx = np.where(above, (1.0 - th * th) / np.where(above, th, 1.0), 0.0)
    beta = 2.0 / (1.0 + np.exp(-y))
    return np.asarray(dg, np.float64) * dgdx, np.asarray(dbeta, np.float64) * beta * (1.0 - 0.5 * beta)


# ----------------------------------------------------------------------------
# Optional short convolution (the width-4 part of the pre-mixer prep).  The
# "complex-kda-1.3B-100B" model card lists a "short convolution of width 4"
# among the layer's parts and says nothing more about it.  Reading taken here:
# a depthwise causal convolution over tokens with one 4-tap filter per channel
# (channels = heads x head dimension), applied to an input before the mixer,
# with zero history before each sequence or document unless the caller gives
# the three inputs that preceded it, optionally followed by SiLU:
#   z_t[c] = sum_{j=0..3} w[c, j] x_{t-3+j}[c],   y_t = z_t or z_t sigmoid(z_t)
# (tap 3 takes the current token).  Written out token by token, per document.
# ----------------------------------------------------------------------------
CONV_WIDTH = 4


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _conv_docs(x, cu_seqlens):
    """Documents of x as (start, stop) row ranges of a [T_total, C] view."""
    x = np.asarray(x, np.float64)
    if cu_seqlens is None:
        B, T, C = x.shape
        return x.reshape(B * T, C), [(b * T, (b + 1) * T) for b in range(B)]
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    return x, [(cu[d], cu[d + 1]) for d in range(len(cu) - 1)]


def short_conv(x, w, cu_seqlens=None, state0=None, silu=False):
    """x: [B, T, C] (sequences), or [T_total, C] with cu_seqlens (documents);
    w: [C, 4]; state0: [nseq, 3, C], the inputs x_{-3}, x_{-2}, x_{-1} before
    each sequence (None: zeros).  Returns (y shaped like x, state_out
    [nseq, 3, C]: each sequence's last three inputs, history included)."""
    xf, docs = _conv_docs(x, cu_seqlens)
    w = np.asarray(w, np.float64)
    C = xf.shape[1]
    y = np.zeros_like(xf)
    st = np.zeros((len(docs), CONV_WIDTH - 1, C))
    for d, (a, b) in enumerate(docs):
        hist = np.zeros((CONV_WIDTH - 1, C)) if state0 is None else np.asarray(state0, np.float64)[d]
        xx = np.concatenate([hist, xf[a:b]], axis=0)   # row i holds x_{i-3}
        for t in range(b - a):
            z = np.zeros(C)
            for j in range(CONV_WIDTH):
                z += w[:, j] * xx[t + j]
            y[a + t] = z * _sigmoid(z) if silu else z
        st[d] = xx[b - a:]
    return y.reshape(np.shape(x)), st


def short_conv_bwd(x, w, dy, cu_seqlens=None, state0=None, silu=False):
    """Reverse mode of short_conv: (dx like x, dw [C, 4], dstate0 [nseq, 3, C])."""
    xf, docs = _conv_docs(x, cu_seqlens)
    dyf = np.asarray(dy, np.float64).reshape(xf.shape)
    w = np.asarray(w, np.float64)
    C = xf.shape[1]
    dx = np.zeros_like(xf)
    dw = np.zeros((C, CONV_WIDTH))
    ds = np.zeros((len(docs), CONV_WIDTH - 1, C))
    for d, (a, b) in enumerate(docs):
        hist = np.zeros((CONV_WIDTH - 1, C)) if state0 is None else np.asarray(state0, np.float64)[d]
        xx = np.concatenate([hist, xf[a:b]], axis=0)
        dxx = np.zeros_like(xx)
        for t in range(b - a):
            z = np.zeros(C)
            for j in range(CONV_WIDTH):
                z += w[:, j] * xx[t + j]
            if silu:
                sg = _sigmoid(z)
                dz = dyf[a + t] * sg * (1.0 + z * (1.0 - sg))
            else:
                dz = dyf[a + t]
            for j in range(CONV_WIDTH):
                dxx[t + j] += w[:, j] * dz
                dw[:, j] += dz * xx[t + j]
        dx[a:b] = dxx[CONV_WIDTH - 1:]
        ds[d] = dxx[:CONV_WIDTH - 1]
    return dx.reshape(np.shape(x)), dw, ds


def short_conv_step(x, w, window, silu=False):
    """One decode step: x [N, C], window [N, 3, C] (the last three inputs).
    Returns (y [N, C], the new window)."""
    x = np.asarray(x, np.float64)
    xx = np.concatenate([np.asarray(window, np.float64), x[:, None, :]], axis=1)
    w = np.asarray(w, np.float64)
    z = np.zeros_like(x)
    for j in range(CONV_WIDTH):
        z += w[None, :, j] * xx[:, j]
    return (z * _sigmoid(z) if silu else z), xx[:, 1:]


# ----------------------------------------------------------------------------
# tensor-level entry points ([B, T, H, D] layout); qk_norm=True runs the
# recurrence on l2norm(q), l2norm(k)
# ----------------------------------------------------------------------------
def fwd(q, k, v, g, s, beta, scale=1.0, h0=None,
        chains: Optional[Sequence] = None, cols: Optional[Sequence[int]] = None, qk_norm: bool = False):
    """Forward over [B,T,H,D] tensors.  Returns (o [B,T,H,DV], ht [B,H,DK,DV]).

    ``chains``: optional list of (b, h) pairs; ``cols``: optional list of value
    columns.  With either given, only those chains / columns are computed and
    the result has shape (o [nchains, T, ncols], ht [nchains, DK, ncols]).
    Every value column evolves on its own (u_j depends only on column j of the
    state and on v_j), so restricting v and h0 to a set of columns gives
    exactly those columns of the full problem."""
    if qk_norm:
        q, k = l2norm(q), l2norm(k)
    B, T, H, DK = q.shape
    if chains is None and cols is None:
        S0 = None if h0 is None else np.asarray(h0, np.float64).reshape(B * H, DK, -1)
        o, ST = fwd_chain_arrays(_chains(q), _chains(k), _chains(v), _chains(g), _chains(s),
                                 np.asarray(beta, np.float64).transpose(0, 2, 1).reshape(B * H, T),
                                 scale, S0)
        return _unchain(o, B, H), ST.reshape(B, H, DK, -1)
    if chains is None:
        chains = [(b, h) for b in range(B) for h in range(H)]
    DV = v.shape[3]
    cols = list(range(DV)) if cols is None else list(cols)
    bi = np.array([c[0] for c in chains]); hi = np.array([c[1] for c in chains])
    sel = lambda x: np.ascontiguousarray(np.asarray(x)[bi, :, hi, :], np.float64)
    vv = np.ascontiguousarray(np.asarray(v)[bi, :, hi, :][:, :, cols], np.float64)
    bb = np.ascontiguousarray(np.asarray(beta)[bi, :, hi], np.float64)
    S0 = None
    if h0 is not None:
        S0 = np.ascontiguousarray(np.asarray(h0)[bi, hi][:, :, cols], np.float64)
    return fwd_chain_arrays(sel(q), sel(k), vv, sel(g), sel(s), bb, scale, S0)


def _drop_lead(x, nd: int) -> np.ndarray:
    x = np.asarray(x)
    return x[0] if x.ndim == nd + 1 else x


def varlen(q, k, v, g, s, beta, cu_seqlens, scale=1.0, h0=None,
           docs: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None,
           cols: Optional[Sequence[int]] = None, qk_norm: bool = False):
    """Packed documents: q etc. are [1, Ttot, H, D] (or [Ttot, H, D]); document
    n covers tokens cu[n]..cu[n+1]-1 and starts from h0[n] (or 0).  Each
    (document, head) is an independent chain.  Returns (o [Ttot, H, DV'],
    ht [N, H, DK, DV']) over the selected docs/heads/cols (o rows of
    unselected documents are NaN)."""
    q, k, v, g, s = (_drop_lead(a, 3) for a in (q, k, v, g, s))
    beta = _drop_lead(beta, 2)
    if qk_norm:
        q, k = l2norm(q), l2norm(k)
    Ttot, H, DK = q.shape
    DV = v.shape[2]
    cu = np.asarray(cu_seqlens, np.int64)
    N = len(cu) - 1
    docs = list(range(N)) if docs is None else list(docs)
    heads = list(range(H)) if heads is None else list(heads)
    cols = list(range(DV)) if cols is None else list(cols)
    o = np.full((Ttot, H, len(cols)), np.nan)
    ht = np.full((N, H, DK, len(cols)), np.nan)
    for n in docs:
        a, b = int(cu[n]), int(cu[n + 1])
        L = b - a
        for h in heads:
            S0 = None if h0 is None else np.asarray(h0, np.float64)[n, h][:, cols][None]
            if L == 0:
                ht[n, h] = 0.0 if S0 is None else S0[0]
                continue
            oc, ST = fwd_chain_arrays(q[None, a:b, h], k[None, a:b, h], v[None, a:b, h][:, :, cols],
                                      g[None, a:b, h], s[None, a:b, h], beta[None, a:b, h],
                                      scale, S0)
            o[a:b, h] = oc[0]
            ht[n, h] = ST[0]
    return o, ht


def decode(q, k, v, g, s, beta, state0, sign0=None, scale=1.0,
           pairs: Optional[Sequence] = None, cols: Optional[Sequence[int]] = None, qk_norm: bool = False):
    """Sequential single-token steps.  q etc. are [steps, N, H, D]; the decode
    state is carried as (state, sign product) with true state
    Diag(sign) * state.  Returns (o [steps, npairs, DV'], true final state
    [npairs, DK, DV'], final sign product [npairs, DK]) for the selected (n, h)
    pairs (default: all, in n-major order)."""
    if qk_norm:
        q, k = l2norm(q), l2norm(k)
    steps, N, H, DK = np.asarray(q).shape
    DV = np.asarray(v).shape[3]
    pairs = [(n, h) for n in range(N) for h in range(H)] if pairs is None else list(pairs)
    cols = list(range(DV)) if cols is None else list(cols)
    ni = np.array([p[0] for p in pairs]); hi = np.array([p[1] for p in pairs])
    sel = lambda x: np.ascontiguousarray(np.asarray(x)[:, ni, hi, :].transpose(1, 0, 2), np.float64)
    P0 = np.ones((len(pairs), DK)) if sign0 is None else np.asarray(sign0, np.float64)[ni, hi]
    st0 = np.asarray(state0, np.float64)[ni, hi][:, :, cols]
    true0 = P0[:, :, None] * st0
    vv = np.ascontiguousarray(np.asarray(v)[:, ni, hi, :][:, :, cols].transpose(1, 0, 2), np.float64)
    bb = np.ascontiguousarray(np.asarray(beta)[:, ni, hi].T, np.float64)
    o, ST = fwd_chain_arrays(sel(q), sel(k), vv, sel(g), sel(s), bb, scale, true0)
    PT = P0 * np.prod(sel(s), axis=1)
    return o.transpose(1, 0, 2), ST, PT


def bwd(q, k, v, g, s, beta, do, scale=1.0, h0=None, dht=None, every=64,
        chains: Optional[Sequence] = None, qk_norm: bool = False):
    """Gradients of L = <do, o> + <dht, ht> for the [B,T,H,D] forward.
    Returns dict with dq, dk, dg [n,T,DK], dv [n,T,DV], dbeta [n,T], dh0
    [n,DK,DV] over the selected (b, h) chains (default: all, b-major)."""
    B, T, H, DK = np.asarray(q).shape
    if chains is None:
        chains = [(b, h) for b in range(B) for h in range(H)]
    bi = np.array([c[0] for c in chains]); hi = np.array([c[1] for c in chains])
    sel = lambda x: np.ascontiguousarray(np.asarray(x)[bi, :, hi, :], np.float64)
    bb = np.ascontiguousarray(np.asarray(beta)[bi, :, hi], np.float64)
    S0 = None if h0 is None else np.ascontiguousarray(np.asarray(h0)[bi, hi], np.float64)
    dST = None if dht is None else np.ascontiguousarray(np.asarray(dht)[bi, hi], np.float64)
    if qk_norm:   # gradients reach the raw q, k through the normalisation
        qr, kr = sel(q), sel(k)
        r = bwd_chain_arrays(l2norm(qr), l2norm(kr), sel(v), sel(g), sel(s), bb, sel(do), scale, S0, dST, every)
        r["dq"], r["dk"] = l2norm_bwd(qr, r["dq"]), l2norm_bwd(kr, r["dk"])
    else:
        r = bwd_chain_arrays(sel(q), sel(k), sel(v), sel(g), sel(s), bb, sel(do), scale, S0, dST, every)
    r["dh0"] = r.pop("dS0")
    return r
