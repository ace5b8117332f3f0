"""Segmented state pass (chunk-parallel scan over long chains) on the GPU.

Per chunk the state map is affine, S' = A_c S + B_c, and every column of S
evolves on its own (the column independence the oracle pins), so a chain
can be cut into segments whose maps are built in parallel and chained by a
scan.  These tests force segments of 16 chunks (1024 tokens) and compare
against the oracle, against the whole-chain pass, and through the backward
(which reads the forward's checkpoints, written by both segment phases).

With the workload's gates (log|alpha| about -0.8 per token) a chain forgets
its state within a chunk, so a segment's map P_s underflows to zero and the
scan is trivially exact.  The inputs here therefore keep a long memory:
log|alpha| and beta scaled down (by 1e-3 and 0.05) so that P_s over 1024
tokens stays of order 0.1-1, with the signs unchanged.  The sharp check is
segmented against whole-chain on the GPU (they differ only by the fp32
scan's rounding); both are also held to the oracle."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu

# against the oracle: the contract bounds, forward and backward (bf16
# records round W once and Qh, KbT, M in hi/lo pairs; a long memory carries
# that rounding further than the workload's gates do)
TOL = {"f32": 1e-4, "bf16": 1e-2}
# segmented against whole-chain: the scan's fp32 rounding only (forward
# outputs and checkpoints; gradients computed from either set of checkpoints)
SEG_VS_WHOLE = 2e-5
GRAD_SEG_VS_WHOLE = 1e-4


def long_memory(tok):
    """Scale log|alpha| by 1e-3 and beta by 0.05 (in place; signs kept)."""
    tok.g *= np.float32(1e-3)
    tok.beta *= np.float32(0.05)
    return tok


@pytest.fixture
def segments():
    """Run the test body with the segment length forced to 16 chunks."""
    from gated_delta_rule_sign_amd import ckda
    ckda.set_segment_chunks(16)
    yield ckda
    ckda.set_segment_chunks(0)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128), ("f32", 32, 128)])
def test_segmented_varlen_forward(segments, dtype, DK, DV):
    torch = require_gpu()
    ckda = segments
    import torch as T_
    # 3300 tokens: 52 chunks, 4 segments (16, 16, 16, 4); 2100: 33 chunks, 3
    # segments; 1030: 17 chunks, 2 segments; the rest stay whole
    lens = [3300, 100, 0, 2100, 1, 1030, 64]
    banner(f"segmented varlen fwd {dtype} DK={DK} DV={DV} lens={lens}")
    cu = I.cu_from_lengths(lens)
    Tt, H, N = int(cu[-1]), 2, len(lens)
    rng = np.random.default_rng(31)
    tok = long_memory(I.draw_tokens(rng, (Tt,), H, DK, DV, dtype))
    h0 = I.draw_state(rng, (N, H, DK, DV), 0.3)
    d = tok_to_dev(tok)
    cu_t = T_.from_numpy(cu)
    o, ht = ckda.fwd_varlen(**d, cu_seqlens=cu_t, scale=0.9, h0=dev_tensor(h0))
    ckda.set_segment_chunks(-1)
    o_w, ht_w = ckda.fwd_varlen(**d, cu_seqlens=cu_t, scale=0.9, h0=dev_tensor(h0))
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.varlen(**tok.f64(), cu_seqlens=cu, scale=0.9, h0=h0.astype(np.float64))
    e_o, e_h = rel_max(host(o), o_ref), rel_max(host(ht), ht_ref)
    e_ow, e_hw = rel_max(host(o), host(o_w)), rel_max(host(ht), host(ht_w))
    print(f"  vs oracle: o {e_o:.2e}  ht {e_h:.2e};  vs whole chains: o {e_ow:.2e}  ht {e_hw:.2e}")
    assert e_o < TOL[dtype]
    assert e_h < TOL[dtype]
    assert e_ow < SEG_VS_WHOLE
    assert e_hw < SEG_VS_WHOLE


@pytest.mark.parametrize("dtype,DK,DV,T", [("f32", 64, 64, 2500), ("bf16", 128, 128, 1500)])
def test_segmented_forward_and_backward(segments, dtype, DK, DV, T):
    """Equal-length chains cut into segments; the backward consumes the
    checkpoints both segment phases write."""
    torch = require_gpu()
    ckda = segments
    B, H = 2, 2
    banner(f"segmented fwd+bwd {dtype} B={B} T={T} H={H} DK={DK} DV={DV}")
    w = I.make_forward(B, T, H, DK, DV, dtype, seed=37 + T, h0_std=0.3)
    long_memory(w.tok)
    rng = np.random.default_rng(T)
    do = I.to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0)
    o, ht, hc = ckda.fwd(**d, scale=0.8, h0=h0, want_ckpt=True)
    ckda.set_segment_chunks(-1)
    o_w, ht_w, hc_w = ckda.fwd(**d, scale=0.8, h0=h0, want_ckpt=True)
    r = ckda.bwd(**d, h_ckpt=hc, do=dev_tensor(do), scale=0.8, h0=h0)
    torch.cuda.synchronize()
    f = w.tok.f64()
    o_ref, ht_ref = oracle.fwd(**f, scale=0.8, h0=w.h0.astype(np.float64))
    print(f"  vs oracle: o {rel_max(host(o), o_ref):.2e}; vs whole chains: o {rel_max(host(o), host(o_w)):.2e} "
          f"ckpt {rel_max(host(hc), host(hc_w)):.2e}")
    assert rel_max(host(o), o_ref) < TOL[dtype]
    assert rel_max(host(ht), ht_ref) < TOL[dtype]
    assert rel_max(host(o), host(o_w)) < SEG_VS_WHOLE
    assert rel_max(host(hc), host(hc_w)) < SEG_VS_WHOLE
    ref = oracle.bwd(**f, do=I.widen(do), scale=0.8, h0=w.h0.astype(np.float64))
    chains = [(b, h) for b in range(B) for h in range(H)]
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        g = host(r[name])
        g = g[bi, :, hi] if g.ndim == 3 else g[bi, :, hi, :]
        e = rel_max(g, ref[name])
        print(f"  {name}: {e:.2e}")
        assert e < TOL[dtype], (name, e)


def test_segmented_varlen_backward(segments):
    torch = require_gpu()
    ckda = segments
    import torch as T_
    dtype, DK, DV = "bf16", 128, 128
    lens = [1100, 2200, 5]
    banner(f"segmented varlen fwd+bwd {dtype} lens={lens}")
    cu = I.cu_from_lengths(lens)
    Tt, H, N = int(cu[-1]), 2, len(lens)
    rng = np.random.default_rng(41)
    tok = long_memory(I.draw_tokens(rng, (Tt,), H, DK, DV, dtype))
    h0 = I.draw_state(rng, (N, H, DK, DV), 0.3)
    do = I.to_storage(rng.standard_normal((Tt, H, DV)), dtype)
    d = tok_to_dev(tok)
    cu_t = T_.from_numpy(cu)
    o, ht, hc = ckda.fwd_varlen(**d, cu_seqlens=cu_t, h0=dev_tensor(h0), want_ckpt=True)
    r = ckda.bwd_varlen(**d, cu_seqlens=cu_t, h_ckpt=hc, do=dev_tensor(do), h0=dev_tensor(h0))
    ckda.set_segment_chunks(-1)
    o_w, ht_w, hc_w = ckda.fwd_varlen(**d, cu_seqlens=cu_t, h0=dev_tensor(h0), want_ckpt=True)
    r_w = ckda.bwd_varlen(**d, cu_seqlens=cu_t, h_ckpt=hc_w, do=dev_tensor(do), h0=dev_tensor(h0))
    torch.cuda.synchronize()
    # chunk j of document n sits in slot cu[n] // 64 + n + j; other slots stay unwritten
    used = [int(cu[n]) // 64 + n + j for n in range(N) for j in range((lens[n] + 63) // 64)]
    e = rel_max(host(hc)[used], host(hc_w)[used])
    print(f"  checkpoints vs whole chains: {e:.2e}")
    assert e < SEG_VS_WHOLE
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        e = rel_max(host(r[name]), host(r_w[name]))
        print(f"  {name} from segmented vs whole-chain checkpoints: {e:.2e}")
        assert e < GRAD_SEG_VS_WHOLE, (name, e)
    f = tok.f64()
    dof = I.widen(do)
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = {k: f[k][a:b][None] for k in ("q", "k", "v", "g", "s", "beta")}
        ref = oracle.bwd(**sl, do=dof[a:b][None], h0=h0[n][None].astype(np.float64))
        for name in ("dq", "dk", "dg"):
            e = rel_max(host(r[name])[a:b], np.moveaxis(ref[name], 0, 1))
            print(f"  doc {n} {name} vs oracle: {e:.2e}")
            assert e < TOL[dtype], (n, name, e)
        assert rel_max(host(r["dh0"])[n], ref["dh0"].reshape(H, DK, DV)) < TOL[dtype]


def test_long_64k_sampled():
    """long_64k at full size (one 65,536-token sequence, 16 heads, d = 128,
    bf16) with the automatic state-pass plan, as bench.py times it (the cost
    model segments it): sampled heads and value columns against the oracle,
    and the whole output against the whole-chain pass."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner("fwd long_64k full size, automatic plan, sampled")
    w = I.make_workload("long_64k")
    d = tok_to_dev(w.tok)
    ckda.set_segment_chunks(0)
    o, ht, _ = ckda.fwd(**d)
    ckda.set_segment_chunks(-1)
    try:
        o_w, ht_w, _ = ckda.fwd(**d)
    finally:
        ckda.set_segment_chunks(0)
    torch.cuda.synchronize()
    e_w = rel_max(host(o), host(o_w))
    print(f"  o vs whole chains: {e_w:.2e}")
    assert e_w < SEG_VS_WHOLE
    o = host(o); ht = host(ht)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    hi = [0, 9, 15]
    cols = [0, 45, 64, 127]
    # the sampled heads only, widened from storage ([1, T, 3, D])
    sub = {k: I.widen(getattr(w.tok, k)[:, :, hi]) for k in ("q", "k", "v", "g", "s")}
    sub["beta"] = w.tok.beta[:, :, hi].astype(np.float64)
    o_ref, ht_ref = oracle.fwd(**sub, cols=cols)
    e_o = rel_max(o[0][:, hi, :][:, :, cols].transpose(1, 0, 2), o_ref)
    e_h = rel_max(ht[0, hi][:, :, cols], ht_ref)
    print(f"  long_64k max|diff|/rms: o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < TOL["bf16"] and e_h < TOL["bf16"]


@pytest.mark.parametrize("dtype,DK,DV,T", [("f32", 64, 64, 2500), ("bf16", 128, 128, 3300), ("f32", 32, 128, 1100)])
def test_segmented_reverse_pass(dtype, DK, DV, T):
    """The backward's reverse (dS) pass cut into segments of 16 chunks (the
    map G' = A'_c G + B'_c is affine with independent value columns, as in
    the forward): the same checkpoints, gradients with segments against
    gradients with whole chains, and both against the oracle."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    B, H = 2, 2
    banner(f"segmented reverse pass {dtype} B={B} T={T} H={H} DK={DK} DV={DV}")
    w = I.make_forward(B, T, H, DK, DV, dtype, seed=53 + T, h0_std=0.3)
    long_memory(w.tok)
    rng = np.random.default_rng(T + 7)
    do_st = I.to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    do = dev_tensor(do_st)
    dht = rng.standard_normal((B, H, DK, DV)).astype(np.float32)
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0)
    try:
        ckda.set_segment_chunks(-1)
        _, _, hc = ckda.fwd(**d, scale=0.8, h0=h0, want_ckpt=True)
        r_w = ckda.bwd(**d, h_ckpt=hc, do=do, scale=0.8, h0=h0, dht=dev_tensor(dht))
        ckda.set_segment_chunks(16)
        # the binding sizes the workspace for given checkpoints (segment
        # buffers in the checkpoint room's place); the full size puts them
        # after that room: same plan, same results
        r = ckda.bwd(**d, h_ckpt=hc, do=do, scale=0.8, h0=h0, dht=dev_tensor(dht))
        ws_full = torch.empty(ckda.bwd_workspace_bytes(B, T, H, DK, DV), dtype=torch.uint8, device="cuda:0")
        r_full = ckda.bwd(**d, h_ckpt=hc, do=do, scale=0.8, h0=h0, dht=dev_tensor(dht), workspace=ws_full)
    finally:
        ckda.set_segment_chunks(0)
    torch.cuda.synchronize()
    assert ckda.bwd_workspace_bytes(B, T, H, DK, DV, ckpt_given=True) < ws_full.numel()
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(r[name], r_full[name]), name
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        e = rel_max(host(r[name]), host(r_w[name]))
        print(f"  {name} segmented vs whole chains: {e:.2e}")
        assert e < GRAD_SEG_VS_WHOLE, (name, e)
    f = w.tok.f64()
    ref = oracle.bwd(**f, do=I.widen(do_st), scale=0.8, h0=w.h0.astype(np.float64), dht=dht.astype(np.float64))
    chains = [(b, h) for b in range(B) for h in range(H)]
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        g = host(r[name])
        g = g[bi, :, hi] if g.ndim == 3 else g[bi, :, hi, :]
        e = rel_max(g, ref[name])
        print(f"  {name} vs oracle: {e:.2e}")
        assert e < TOL[dtype], (name, e)
    assert rel_max(host(r["dh0"]).reshape(B * H, DK, DV), ref["dh0"]) < TOL[dtype]
