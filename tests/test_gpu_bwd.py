"""Backward on the GPU against the oracle's reverse-mode token recurrence
(itself pinned to central finite differences)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}
NAMES = ("dq", "dk", "dv", "dg", "dbeta")


def gpu_bwd(w, do, dht=None, scale=1.0):
    import torch
    from gated_delta_rule_sign_amd import ckda
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0) if w.h0 is not None else None
    _, _, hc = ckda.fwd(**d, scale=scale, h0=h0, want_ckpt=True)
    r = ckda.bwd(**d, h_ckpt=hc, do=dev_tensor(do), scale=scale, h0=h0,
                 dht=None if dht is None else dev_tensor(dht))
    torch.cuda.synchronize()
    return r


CASES = [
    ("f32", 1, 130, 2, 64, 64),
    ("f32", 2, 64, 1, 32, 128),
    ("bf16", 1, 200, 2, 128, 128),
    ("f32", 1, 1, 1, 32, 32),
    ("f32", 1, 96, 1, 128, 32),
    # whole chunks with several sequences and heads: the gradients go straight
    # into their [B, T, H, D] places
    ("f32", 2, 128, 2, 64, 64),
    ("bf16", 2, 128, 2, 128, 128),
]


@pytest.mark.parametrize("dtype,B,T,H,DK,DV", CASES)
def test_backward_small(dtype, B, T, H, DK, DV):
    require_gpu()
    banner(f"bwd {dtype} B={B} T={T} H={H} DK={DK} DV={DV}")
    w = I.make_forward(B, T, H, DK, DV, dtype, seed=31 + T, h0_std=0.3)
    rng = np.random.default_rng(T)
    do = I.to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    dht = rng.standard_normal((B, H, DK, DV)).astype(np.float32)
    r = gpu_bwd(w, do, dht, scale=0.7)
    f = w.tok.f64()
    ref = oracle.bwd(**f, do=I.widen(do), scale=0.7, h0=w.h0.astype(np.float64), dht=dht.astype(np.float64))
    chains = [(b, h) for b in range(B) for h in range(H)]
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    design = 1e-4 if dtype == "f32" else 1e-3
    for name in NAMES:
        g = host(r[name])
        g = g[bi, :, hi] if g.ndim == 3 else g[bi, :, hi, :]
        e = rel_max(g, ref[name])
        print(f"  {name}: {e:.2e}")
        assert e < design, (name, e)
    e = rel_max(host(r["dh0"]).reshape(B * H, DK, DV), ref["dh0"])
    print(f"  dh0: {e:.2e}")
    assert e < design


def test_layer_bwd_sampled():
    """B=8, T=4096, H=16, d=128 bf16 with a bf16 upstream gradient, plus a
    nonzero initial state and final-state gradient; whole backward on the GPU,
    four (sequence, head) chains (the first, the last and two inside) against
    the oracle, dh0 included."""
    require_gpu()
    banner("bwd layer_bwd full size, sampled")
    w = I.make_workload("layer_bwd")
    B, T, H, DK = w.tok.q.shape
    DV = w.tok.v.shape[-1]
    rng = np.random.default_rng(4096)
    h0 = I.draw_state(rng, (B, H, DK, DV), 0.02)
    dht = (0.05 * rng.standard_normal((B, H, DK, DV))).astype(np.float32)
    w.h0 = h0
    r = gpu_bwd(w, w.do, dht)
    for name in NAMES + ("dh0",):
        assert np.isfinite(r[name].cpu().numpy()).all(), name
    chains = [(0, 0), (1, 3), (6, 14), (B - 1, H - 1)]
    f = w.tok.f64()
    ref = oracle.bwd(**f, do=I.widen(w.do), h0=h0.astype(np.float64), dht=dht.astype(np.float64),
                     chains=chains)
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    for name in NAMES:
        g = host(r[name])
        g = g[bi, :, hi] if g.ndim == 3 else g[bi, :, hi, :]
        e = rel_max(g, ref[name])
        print(f"  layer_bwd {name}: {e:.2e}")
        assert e < TOL["bf16"], (name, e)
    e = rel_max(host(r["dh0"])[bi, hi], ref["dh0"])
    print(f"  layer_bwd dh0: {e:.2e}")
    assert e < TOL["bf16"]


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_backward_recomputes_checkpoints(dtype, DK, DV):
    """h_ckpt = None: the backward runs the forward itself for the chunk
    checkpoints; with the same (whole-chain) forward the gradients equal those
    from the caller's checkpoints, equal-length and varlen."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    import torch as T_
    banner(f"bwd recomputed checkpoints {dtype} DK={DK} DV={DV}")
    w = I.make_forward(2, 150, 2, DK, DV, dtype, seed=61, h0_std=0.3)
    rng = np.random.default_rng(62)
    do = dev_tensor(I.to_storage(rng.standard_normal((2, 150, 2, DV)), dtype))
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0)
    try:
        ckda.set_segment_chunks(-1)
        _, _, hc = ckda.fwd(**d, h0=h0, want_ckpt=True)
        r1 = ckda.bwd(**d, h_ckpt=hc, do=do, h0=h0)
        r2 = ckda.bwd(**d, h_ckpt=None, do=do, h0=h0)
        lens = [0, 130, 1, 170]
        cu = I.cu_from_lengths(lens)
        Tt = int(cu[-1])
        tok = I.draw_tokens(rng, (Tt,), 2, DK, DV, dtype)
        dv_ = tok_to_dev(tok)
        dov = dev_tensor(I.to_storage(rng.standard_normal((Tt, 2, DV)), dtype))
        cu_t = T_.from_numpy(cu)
        _, _, hcv = ckda.fwd_varlen(**dv_, cu_seqlens=cu_t, want_ckpt=True)
        v1 = ckda.bwd_varlen(**dv_, cu_seqlens=cu_t, h_ckpt=hcv, do=dov)
        v2 = ckda.bwd_varlen(**dv_, cu_seqlens=cu_t, h_ckpt=None, do=dov)
    finally:
        ckda.set_segment_chunks(0)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert np.array_equal(host(r1[name]), host(r2[name])), name
        assert np.array_equal(host(v1[name]), host(v2[name])), name
