"""The optional gate map (CKDA_GATE_MAP) on the GPU: g and beta carry the
gate and beta pre-activations x and y, mapped inside the kernels' loads.
Against the oracle's gate_map composed with its forward / decode, and for the
backward with the oracle's reverse mode followed by gate_map_bwd (the map's
own pins, and the reading it takes of the paper page's section 3 "CKDA."
paragraph, are in tests/test_oracle_pins.py; its floor is parity unpinned)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def mapped(tok, x, y):
    """f64 token dict with the mapped gates in place of g, s, beta."""
    f = tok.f64()
    g, s, beta = oracle.gate_map(x, y)
    f.update(g=g, s=s, beta=beta)
    return f


def dev_inputs(tok, x, y):
    return dict(q=dev_tensor(tok.q), k=dev_tensor(tok.k), v=dev_tensor(tok.v), g=dev_tensor(x), s=None,
                beta=dev_tensor(y))


@pytest.mark.parametrize("dtype,B,T,H,DK,DV,gate", [("f32", 1, 200, 2, 64, 64, "channel"),
                                                    ("bf16", 2, 130, 2, 128, 128, "channel"),
                                                    ("f32", 1, 96, 2, 32, 128, "head"),
                                                    ("bf16", 1, 150, 2, 128, 64, "head")])
def test_gate_map_forward_and_backward(dtype, B, T, H, DK, DV, gate):
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner(f"gate map fwd+bwd {dtype} B={B} T={T} H={H} DK={DK} DV={DV} gate={gate}")
    rng = np.random.default_rng(91 + T)
    tok = I.draw_tokens(rng, (B, T), H, DK, DV, dtype)
    gshape = (B, T, H) if gate == "head" else (B, T, H, DK)
    x, y = I.draw_gate_preacts(rng, gshape, (B, T, H))
    h0 = I.draw_state(rng, (B, H, DK, DV), 0.3)
    do = I.to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    dht = rng.standard_normal((B, H, DK, DV)).astype(np.float32)
    d = dev_inputs(tok, x, y)
    o, ht, hc = ckda.fwd(**d, scale=0.7, h0=dev_tensor(h0), want_ckpt=True, gate_map=True)
    r = ckda.bwd(**d, h_ckpt=hc, do=dev_tensor(do), scale=0.7, h0=dev_tensor(h0), dht=dev_tensor(dht),
                 gate_map=True)
    torch.cuda.synchronize()
    f = mapped(tok, x, y)
    if gate == "head":   # one gate per head is the channel gate with equal entries
        f["g"] = np.repeat(f["g"][..., None], DK, axis=-1)
        f["s"] = np.repeat(f["s"][..., None], DK, axis=-1)
    o_ref, ht_ref = oracle.fwd(**f, scale=0.7, h0=h0.astype(np.float64))
    e_o, e_h = rel_max(host(o), o_ref), rel_max(host(ht), ht_ref)
    print(f"  o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < TOL[dtype] and e_h < TOL[dtype]
    ref = oracle.bwd(**f, do=I.widen(do), scale=0.7, h0=h0.astype(np.float64), dht=dht.astype(np.float64))
    chains = [(b, h) for b in range(B) for h in range(H)]
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    # the chain rule through the map, on the oracle's side
    dg_ref = ref["dg"].sum(axis=-1) if gate == "head" else ref["dg"]
    xs = x[bi, :, hi] if gate == "head" else x[bi, :, hi, :]
    dx_ref, dy_ref = oracle.gate_map_bwd(xs, y[bi, :, hi], dg_ref, ref["dbeta"])
    design = 1e-4 if dtype == "f32" else 1e-3
    got = {}
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        a = host(r[name])
        got[name] = a[bi, :, hi] if a.ndim == 3 else a[bi, :, hi, :]
    for name, want in (("dq", ref["dq"]), ("dk", ref["dk"]), ("dv", ref["dv"]), ("dbeta", dy_ref)):
        e = rel_max(got[name], want)
        print(f"  {name}: {e:.2e}")
        assert e < design, (name, e)
    # dL/dx = dL/dg times the map's derivative, which reaches about 54 just
    # above the floor (and is 0 on it): dL/dx carries dL/dg's error times
    # that factor, so dL/dx over the derivative is held to the contract
    # tolerance against the oracle's dL/dg, and dL/dx must be exactly 0 on
    # the floor
    fac, _ = oracle.gate_map_bwd(xs, y[bi, :, hi], np.ones_like(xs), np.zeros_like(y[bi, :, hi]))
    on = fac != 0.0
    assert np.all(got["dg"][~on] == 0.0)
    e = rel_max(got["dg"][on] / fac[on], dg_ref[on])
    print(f"  dg (dL/dx over the map's derivative): {e:.2e};  dL/dx itself: {rel_max(got['dg'], dx_ref):.2e}")
    assert e < design, ("dg", e)
    e = rel_max(host(r["dh0"]).reshape(B * H, DK, DV), ref["dh0"])
    print(f"  dh0: {e:.2e}")
    assert e < design


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_gate_map_varlen_forward(dtype, DK, DV):
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner(f"gate map varlen fwd {dtype} DK={DK} DV={DV}")
    lens = [70, 1, 129, 0, 64]
    cu = I.cu_from_lengths(lens)
    Tt, H = int(cu[-1]), 2
    rng = np.random.default_rng(93)
    tok = I.draw_tokens(rng, (Tt,), H, DK, DV, dtype)
    x, y = I.draw_gate_preacts(rng, (Tt, H, DK), (Tt, H))
    h0 = I.draw_state(rng, (len(lens), H, DK, DV), 0.3)
    o, ht = ckda.fwd_varlen(**dev_inputs(tok, x, y), cu_seqlens=torch.from_numpy(cu), scale=0.9,
                            h0=dev_tensor(h0), gate_map=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.varlen(**mapped(tok, x, y), cu_seqlens=cu, scale=0.9, h0=h0.astype(np.float64))
    e_o, e_h = rel_max(host(o), o_ref), rel_max(host(ht), ht_ref)
    print(f"  o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < TOL[dtype] and e_h < TOL[dtype]


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 128), ("bf16", 128, 128)])
def test_gate_map_decode(dtype, DK, DV):
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner(f"gate map decode {dtype} DK={DK} DV={DV}")
    N, H, steps = 3, 2, 12
    rng = np.random.default_rng(94)
    tok = I.decode_steps(95, 0, steps, N, H, DK, DV, dtype)
    x, y = I.draw_gate_preacts(rng, (steps, N, H, DK), (steps, N, H))
    state0 = I.draw_state(rng, (N, H, DK, DV), 0.5)
    state = dev_tensor(state0)
    sp = torch.ones((N, H, DK), dtype=torch.int8, device="cuda:0")
    d = dev_inputs(tok, x, y)
    outs = []
    for t in range(steps):
        outs.append(ckda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], None, d["beta"][t], state, sp,
                                     scale=0.75, gate_map=True))
    torch.cuda.synchronize()
    o = np.stack([host(v) for v in outs])
    o_ref, S_ref, P_ref = oracle.decode(**mapped(tok, x, y), state0=state0.astype(np.float64), scale=0.75)
    true_gpu = sp.cpu().numpy().reshape(N * H, DK, 1).astype(np.float64) * host(state).reshape(N * H, DK, DV)
    e_o, e_s = rel_max(o.reshape(steps, N * H, DV), o_ref), rel_max(true_gpu, S_ref)
    print(f"  o {e_o:.2e}  state {e_s:.2e}")
    assert e_o < TOL[dtype] and e_s < TOL[dtype]
    assert np.array_equal(sp.cpu().numpy().reshape(N * H, DK), P_ref.astype(np.int8))
