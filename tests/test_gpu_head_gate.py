"""Head-scalar signed gate (one g and one s per token and head, the Scalar
Gate of the Complex KDA paper page, section 3) on the GPU.  By definition it
is the channel gate with equal entries, so the oracle runs on the gates
broadcast over the key channels, and the head's dg is the sum over channels
of the channel-gate dg."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu


def channel_gates(f, DK):
    """f64 token dict with head gates [..., H] broadcast to [..., H, DK]."""
    out = dict(f)
    for k in ("g", "s"):
        out[k] = np.repeat(f[k][..., None], DK, axis=-1)
    return out


@pytest.mark.parametrize("dtype,B,T,H,DK,DV", [("f32", 1, 200, 2, 64, 64), ("bf16", 2, 130, 2, 128, 128),
                                               ("f32", 1, 96, 1, 32, 128)])
def test_head_gate_forward_and_backward(dtype, B, T, H, DK, DV):
    torch = require_gpu()
    banner(f"head gate fwd+bwd {dtype} B={B} T={T} H={H} DK={DK} DV={DV}")
    from gated_delta_rule_sign_amd import ckda
    w = I.make_forward(B, T, H, DK, DV, dtype, seed=71 + T, h0_std=0.3, gate="head")
    assert w.tok.g.shape == (B, T, H)
    rng = np.random.default_rng(T)
    do = I.to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    dht = rng.standard_normal((B, H, DK, DV)).astype(np.float32)
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0)
    o, ht, hc = ckda.fwd(**d, scale=0.7, h0=h0, want_ckpt=True)
    r = ckda.bwd(**d, h_ckpt=hc, do=dev_tensor(do), scale=0.7, h0=h0, dht=dev_tensor(dht))
    torch.cuda.synchronize()
    f = channel_gates(w.tok.f64(), DK)
    o_ref, ht_ref = oracle.fwd(**f, scale=0.7, h0=w.h0.astype(np.float64))
    design = 1e-4 if dtype == "f32" else 2e-3
    assert rel_max(host(o), o_ref) < design
    assert rel_max(host(ht), ht_ref) < design
    ref = oracle.bwd(**f, do=I.widen(do), scale=0.7, h0=w.h0.astype(np.float64), dht=dht.astype(np.float64))
    chains = [(b, h) for b in range(B) for h in range(H)]
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    bdesign = 1e-4 if dtype == "f32" else 1e-3
    assert r["dg"].shape == (B, T, H)
    for name in ("dq", "dk", "dv", "dbeta"):
        g = host(r[name])
        g = g[bi, :, hi] if g.ndim == 3 else g[bi, :, hi, :]
        e = rel_max(g, ref[name])
        print(f"  {name}: {e:.2e}")
        assert e < bdesign, (name, e)
    dg = host(r["dg"])[bi, :, hi]                     # [chains, T]
    e = rel_max(dg, ref["dg"].sum(axis=-1))
    print(f"  dg (head): {e:.2e}")
    assert e < bdesign
    assert rel_max(host(r["dh0"]).reshape(B * H, DK, DV), ref["dh0"]) < bdesign


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_head_gate_varlen_forward_and_backward(dtype, DK, DV):
    torch = require_gpu()
    banner(f"head gate varlen {dtype} DK={DK} DV={DV}")
    from gated_delta_rule_sign_amd import ckda
    import torch as T_
    lens = [0, 1, 63, 64, 65, 130, 0, 200]
    cu = I.cu_from_lengths(lens)
    Tt, H, N = int(cu[-1]), 2, len(lens)
    rng = np.random.default_rng(13)
    tok = I.draw_tokens(rng, (Tt,), H, DK, DV, dtype, gate="head")
    h0 = I.draw_state(rng, (N, H, DK, DV), 0.3)
    do = I.to_storage(rng.standard_normal((Tt, H, DV)), dtype)
    d = tok_to_dev(tok)
    cu_t = T_.from_numpy(cu)
    o, ht, hc = ckda.fwd_varlen(**d, cu_seqlens=cu_t, scale=0.9, h0=dev_tensor(h0), want_ckpt=True)
    r = ckda.bwd_varlen(**d, cu_seqlens=cu_t, h_ckpt=hc, do=dev_tensor(do), scale=0.9, h0=dev_tensor(h0))
    torch.cuda.synchronize()
    f = channel_gates(tok.f64(), DK)
    o_ref, ht_ref = oracle.varlen(**f, cu_seqlens=cu, scale=0.9, h0=h0.astype(np.float64))
    design = 1e-4 if dtype == "f32" else 2e-3
    assert rel_max(host(o), o_ref) < design
    assert rel_max(host(ht), ht_ref) < design
    dof = I.widen(do)
    got_dg, ref_dg, got_dk, ref_dk = [], [], [], []
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            continue
        sl = {k: f[k][a:b][None] for k in ("q", "k", "v", "g", "s", "beta")}
        ref = oracle.bwd(**sl, do=dof[a:b][None], scale=0.9, h0=h0[n][None].astype(np.float64))
        got_dg.append(host(r["dg"])[a:b]); ref_dg.append(ref["dg"].sum(axis=-1).T)
        got_dk.append(host(r["dk"])[a:b]); ref_dk.append(np.moveaxis(ref["dk"], 0, 1))
    bdesign = 1e-4 if dtype == "f32" else 1e-3
    assert rel_max(np.concatenate(got_dk), np.concatenate(ref_dk)) < bdesign
    assert rel_max(np.concatenate(got_dg), np.concatenate(ref_dg)) < bdesign


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_gate_decode(dtype):
    torch = require_gpu()
    banner(f"head gate decode {dtype}")
    from gated_delta_rule_sign_amd import ckda
    N, H, DK, DV, steps = 3, 2, 64, 128, 5
    rng = np.random.default_rng(17)
    tok = I.draw_tokens(rng, (steps, N), H, DK, DV, dtype, gate="head")
    state0 = I.draw_state(rng, (N, H, DK, DV), 0.3)
    d = tok_to_dev(tok)
    state = dev_tensor(state0)
    sp = torch.ones((N, H, DK), dtype=torch.int8, device="cuda:0")
    outs = []
    for t in range(steps):
        outs.append(host(ckda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["s"][t],
                                          d["beta"][t], state, sp, scale=0.8)))
    torch.cuda.synchronize()
    f = channel_gates(tok.f64(), DK)
    o_ref, ST, PT = oracle.decode(**f, state0=state0.astype(np.float64), scale=0.8)
    design = 1e-4 if dtype == "f32" else 2e-3
    assert rel_max(np.stack(outs).reshape(steps, N * H, DV), o_ref) < design
    true_state = (host(sp).astype(np.float64)[..., None] * host(state)).reshape(N * H, DK, DV)
    assert rel_max(true_state, ST) < design
    assert np.array_equal(host(sp).reshape(N * H, DK), PT.astype(np.int8))


def test_layer_head_gate_sampled():
    """layer_bf16_head_gate at full size (B=8, T=4096, H=16, d=128, one gate
    per token and head), as bench.py times it: sampled chains and value
    columns against the oracle on the broadcast gates."""
    torch = require_gpu()
    banner("fwd layer_bf16_head_gate full size, sampled")
    from gated_delta_rule_sign_amd import ckda
    w = I.make_workload("layer_bf16_head_gate")
    o, ht, _ = ckda.fwd(**tok_to_dev(w.tok))
    torch.cuda.synchronize()
    o = host(o); ht = host(ht)
    chains = [(0, 3), (4, 11), (7, 15)]
    cols = [0, 31, 64, 127]
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    # the sampled chains only ([2 or 3, T, 1, D]), gates broadcast over the channels
    tk = w.tok
    sub = {k: I.widen(getattr(tk, k)[bi, :, hi])[:, :, None] for k in ("q", "k", "v")}
    sub["beta"] = tk.beta[bi, :, hi].astype(np.float64)[:, :, None]
    for k in ("g", "s"):
        sub[k] = np.repeat(getattr(tk, k)[bi, :, hi].astype(np.float64)[:, :, None, None], 128, axis=-1)
    o_ref, ht_ref = oracle.fwd(**sub, cols=cols)
    e_o = rel_max(o[bi, :, hi, :][:, :, cols], o_ref)
    e_h = rel_max(ht[bi, hi][:, :, cols], ht_ref)
    print(f"  head gate max|diff|/rms: o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < 1e-2 and e_h < 1e-2
