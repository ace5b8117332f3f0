"""Seeded synthetic inputs for the Complex KDA (CKDA) recurrence.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It holds no part of the recurrence itself: it only draws random
tensors with the shapes and distributions of the workloads below and rounds
them once to the storage dtype.

Workloads (the mixer of the 1.36B model card: 16 heads of dimension 128,
trained context 4096 -- "complex-kda-1.3B-100B" model card, Architecture):

* ``tiny_fp32``    B=1, T=256, H=2, dk=dv=32, fp32, zero initial state.
* ``layer_bf16``   B=8, T=4096, H=16, dk=dv=128, bf16 q/k/v, zero initial state.
* ``layer_bwd``    as ``layer_bf16`` plus an upstream gradient do ~ N(0,1) in bf16.
* ``decode_b256``  256 sequences x 16 heads, 512 single-token steps, fp32
                   state0 ~ 0.02*N(0,1).
* ``varlen_64k``   65536 packed tokens in 16 documents (Dirichlet(1) split,
                   each >= 256 tokens), per-document state0 ~ 0.02*N(0,1).

Per token and head: q, k ~ N(0,1) then L2-normalised over the channel axis
(unit keys, as the delta-rule analysis on the paper page, section 2 "Linear
RNNs", assumes); v ~ N(0,1); beta ~ U[0,2]; the signed gate alpha = s*|alpha|
with |alpha| = exp(-softplus(z)), z ~ N(0,1), and s = -1 with probability 0.3
per token and channel.  The gate is handed over as g = log|alpha| (fp32) and
s (int8 +-1), the log-magnitude / sign split described on the model card
("complex-kda-1.3B-100B", first section).

With qk="raw" (inputs for the in-path normalisation of q and k) q and k are
not normalised: each (token, head) row is N(0,1) times a factor exp(N(0,1)),
so row norms spread over about two decades around sqrt(DK).

Values are drawn in float64 and rounded once, round-to-nearest-even, to the
storage dtype.  bf16 tensors are kept as uint16 bit patterns (numpy has no
bfloat16); ``widen`` returns the exact float64 value of any stored tensor.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_BASE = 1000

WORKLOADS = {
    "tiny_fp32": dict(index=0, B=1, T=256, H=2, DK=32, DV=32, dtype="f32"),
    "layer_bf16": dict(index=1, B=8, T=4096, H=16, DK=128, DV=128, dtype="bf16"),
    "layer_bwd": dict(index=2, B=8, T=4096, H=16, DK=128, DV=128, dtype="bf16"),
    "decode_b256": dict(index=3, N=256, H=16, DK=128, DV=128, steps=512, dtype="bf16"),
    "varlen_64k": dict(index=4, T=65536, ndocs=16, min_len=256, H=16, DK=128, DV=128,
                       dtype="bf16"),
    # layer_bf16 with one signed gate per (token, head): the head-scalar gate
    "layer_bf16_head_gate": dict(index=5, B=8, T=4096, H=16, DK=128, DV=128, dtype="bf16",
                                 gate="head"),
    # layer_bf16 with raw q, k that the path L2-normalises itself
    "layer_bf16_qk_norm": dict(index=6, B=8, T=4096, H=16, DK=128, DV=128, dtype="bf16",
                               qk="raw"),
    # one long sequence: 16 (sequence, head) chains of 1024 chunks
    "long_64k": dict(index=7, B=1, T=65536, H=16, DK=128, DV=128, dtype="bf16"),
}


# ----------------------------------------------------------------------------
# rounding helpers (storage formats only)
# ----------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values once (RNE) to bfloat16; returns float64 values."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    del m
    # bfloat16 keeps 8 significant bits; below 2**-126 it is subnormal with a
    # fixed quantum of 2**-133.
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def bf16_bits(x64: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float64 values that are already bf16-exact."""
    f32 = np.ascontiguousarray(x64, dtype=np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(round_bf16(x64))
    if dtype == "f32":
        return x64.astype(np.float32)
    raise ValueError(dtype)


def widen(arr: np.ndarray, dtype: Optional[str] = None) -> np.ndarray:
    """Exact float64 value of a stored tensor (bf16 given as uint16 bits)."""
    if arr.dtype == np.uint16:
        return bf16_to_f64(arr)
    return arr.astype(np.float64)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------
def _softplus(z: np.ndarray) -> np.ndarray:
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _l2norm_last(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


@dataclasses.dataclass
class TokenInputs:
    """Per-token tensors, layout [..., H, D] with the token axes first."""
    q: np.ndarray      # storage dtype (float32 or bf16 bits), [..., H, DK]
    k: np.ndarray      # [..., H, DK]
    v: np.ndarray      # [..., H, DV]
    g: np.ndarray      # float32 log|alpha| <= 0, [..., H, DK] (head gate: [..., H])
    s: np.ndarray      # int8 +-1, same shape as g
    beta: np.ndarray   # float32 in [0, 2], [..., H]
    dtype: str

    def f64(self):
        return dict(q=widen(self.q), k=widen(self.k), v=widen(self.v),
                    g=self.g.astype(np.float64), s=self.s.astype(np.float64),
                    beta=self.beta.astype(np.float64))


def _raw_rows(rng: np.random.Generator, shp: tuple) -> np.ndarray:
    return rng.standard_normal(shp) * np.exp(rng.standard_normal(shp[:-1] + (1,)))


def draw_tokens(rng: np.random.Generator, lead: tuple, H: int, DK: int, DV: int,
                dtype: str, p_neg: float = 0.3, gate: str = "channel", qk: str = "unit") -> TokenInputs:
    """Draw order: z, sign mask, q, k, v, beta.  gate="head" draws one g
    and one s per (token, head) instead of per channel; qk="raw" leaves q
    and k unnormalised with spread row norms."""
    shp_k = tuple(lead) + (H, DK)
    shp_v = tuple(lead) + (H, DV)
    shp_g = shp_k if gate == "channel" else tuple(lead) + (H,)
    z = rng.standard_normal(shp_g)
    g = (-_softplus(z)).astype(np.float32)
    del z
    neg = rng.random(shp_g) < p_neg
    s = np.where(neg, -1, 1).astype(np.int8)
    del neg
    if qk == "raw":
        q = to_storage(_raw_rows(rng, shp_k), dtype)
        k = to_storage(_raw_rows(rng, shp_k), dtype)
    else:
        q = to_storage(_l2norm_last(rng.standard_normal(shp_k)), dtype)
        k = to_storage(_l2norm_last(rng.standard_normal(shp_k)), dtype)
    v = to_storage(rng.standard_normal(shp_v), dtype)
    beta = (2.0 * rng.random(tuple(lead) + (H,))).astype(np.float32)
    return TokenInputs(q=q, k=k, v=v, g=g, s=s, beta=beta, dtype=dtype)


def draw_state(rng: np.random.Generator, shape: tuple, std: float = 0.02) -> np.ndarray:
    return (std * rng.standard_normal(shape)).astype(np.float32)


def dirichlet_lengths(rng: np.random.Generator, total: int, ndocs: int, min_len: int) -> np.ndarray:
    """Document lengths: min_len + floor(w_i * (total - ndocs*min_len)),
    w ~ Dirichlet(1,...,1); the rounding remainder goes to the last document."""
    w = rng.dirichlet(np.ones(ndocs))
    free = total - ndocs * min_len
    lens = min_len + np.floor(w * free).astype(np.int64)
    lens[-1] += total - int(lens.sum())
    return lens


def cu_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return cu


def draw_gate_preacts(rng: np.random.Generator, gshape: tuple, bshape: tuple):
    """Pre-activations for the optional gate map: the gate's x ~ 1.5 N(0,1)
    (|tanh x| spans the floor up to about 1, both signs) and beta's
    y ~ N(0,1), both float32."""
    x = (1.5 * rng.standard_normal(gshape)).astype(np.float32)
    y = rng.standard_normal(bshape).astype(np.float32)
    return x, y


def decode_steps(seed: int, t0: int, t1: int, N: int, H: int, DK: int, DV: int,
                 dtype: str) -> TokenInputs:
    """Token inputs of decode steps t0..t1-1, stacked as [t1-t0, N, H, D].
    Step t draws from its own stream (seed, t), so any range of steps can be
    produced on its own and a short run is a prefix of a long one."""
    parts = [draw_tokens(np.random.default_rng([seed, t]), (N,), H, DK, DV, dtype)
             for t in range(t0, t1)]
    cat = lambda f: np.stack([getattr(p, f) for p in parts])
    return TokenInputs(q=cat("q"), k=cat("k"), v=cat("v"), g=cat("g"), s=cat("s"),
                       beta=cat("beta"), dtype=dtype)


# ----------------------------------------------------------------------------
# named workloads
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    cfg: dict
    tok: TokenInputs
    h0: Optional[np.ndarray] = None          # float32 [B or N, H, DK, DV]
    do: Optional[np.ndarray] = None          # storage dtype [B, T, H, DV]
    cu_seqlens: Optional[np.ndarray] = None  # int32 [ndocs+1]


def make_forward(B, T, H, DK, DV, dtype, seed, with_do=False, h0_std=None, gate="channel",
                 qk="unit") -> Workload:
    rng = np.random.default_rng(seed)
    tok = draw_tokens(rng, (B, T), H, DK, DV, dtype, gate=gate, qk=qk)
    h0 = draw_state(rng, (B, H, DK, DV), h0_std) if h0_std else None
    do = to_storage(rng.standard_normal((B, T, H, DV)), dtype) if with_do else None
    cfg = dict(B=B, T=T, H=H, DK=DK, DV=DV, dtype=dtype)
    return Workload(name="custom", cfg=cfg, tok=tok, h0=h0, do=do)


def make_workload(name: str, **override) -> Workload:
    """Build a named workload; keyword overrides shrink it (e.g. T=512) while
    keeping the recipe (seed stays that of the named workload unless given)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    seed = cfg.pop("seed", SEED_BASE + cfg["index"])
    rng = np.random.default_rng(seed)
    H, DK, DV, dt = cfg["H"], cfg["DK"], cfg["DV"], cfg["dtype"]
    if name in ("tiny_fp32", "layer_bf16", "layer_bwd", "layer_bf16_head_gate", "layer_bf16_qk_norm", "long_64k"):
        B, T = cfg["B"], cfg["T"]
        tok = draw_tokens(rng, (B, T), H, DK, DV, dt, gate=cfg.get("gate", "channel"),
                          qk=cfg.get("qk", "unit"))
        do = None
        if name == "layer_bwd":
            do = to_storage(rng.standard_normal((B, T, H, DV)), dt)
        return Workload(name=name, cfg=cfg, tok=tok, do=do)
    if name == "decode_b256":
        N, steps = cfg["N"], cfg["steps"]
        state0 = draw_state(rng, (N, H, DK, DV), 0.02)
        tok = decode_steps(seed, 0, steps, N, H, DK, DV, dt)
        return Workload(name=name, cfg=cfg, tok=tok, h0=state0)
    if name == "varlen_64k":
        T, nd, ml = cfg["T"], cfg["ndocs"], cfg["min_len"]
        lens = dirichlet_lengths(rng, T, nd, ml)
        cu = cu_from_lengths(lens)
        tok = draw_tokens(rng, (1, T), H, DK, DV, dt)
        h0 = draw_state(rng, (nd, H, DK, DV), 0.02)
        return Workload(name=name, cfg=cfg, tok=tok, h0=h0, cu_seqlens=cu)
    raise KeyError(name)


def draw_conv(seed: int, x_shape: tuple, C: int, nseq: int, dtype: str, with_state: bool = True):
    """Inputs of the optional short convolution: x ~ N(0,1) shaped x_shape
    (stored in dtype), per-channel taps w [C, 4] ~ U(-1, 1) / 2 (the scale of a
    width-4 filter's default uniform init), a window state0 [nseq, 3, C] ~ N(0,1)
    in dtype (or None), and an upstream gradient dy ~ N(0,1) in float32."""
    rng = np.random.default_rng(seed)
    x = to_storage(rng.standard_normal(x_shape), dtype)
    w = (rng.uniform(-1.0, 1.0, (C, 4)) / 2.0).astype(np.float32)
    s0 = to_storage(rng.standard_normal((nseq, 3, C)), dtype) if with_state else None
    dy = rng.standard_normal(x_shape).astype(np.float32)
    return x, w, s0, dy
