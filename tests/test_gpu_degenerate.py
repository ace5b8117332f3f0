"""Degenerate and extreme inputs of the method on the GPU, against the oracle.

- Gates at the documented edge: the forward factors e^{b_r - b_i} through
  anchors at the middle of each half chunk, so runs of 16 log-gates may sum
  to no less than -80 per channel; the backward anchors at the chunk middle
  and needs 32-token partial sums above -80.  Both edges are run here, on
  half of the channels, the other half keeping ordinary gates.
- beta = 0: nothing is written; the initial state only decays and rotates
  sign (o_t = scale (Diag(alpha_1 ... alpha_t) S0)^T q_t).
- beta = 2 with |alpha| = 1 (g = 0) and random signs: every transition is
  orthogonal (the rotation and reflection cases of the paper page, section 3,
  "CKDA."), the state never decays and T = (I + Diag(beta) A)^-1 Diag(beta)
  reaches its largest entries.
- Zero q and k rows: a zero key writes nothing, a zero query reads exactly
  zero."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu

# contract bounds, max|diff| / RMS of the oracle (fp32 and bf16 inputs)
TOL = {"f32": 1e-4, "bf16": 1e-2}


def run_fwd(w, scale=1.0):
    import torch
    from gated_delta_rule_sign_amd import ckda
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0) if w.h0 is not None else None
    o, ht, hc = ckda.fwd(**d, scale=scale, h0=h0, want_ckpt=True)
    torch.cuda.synchronize()
    return o, ht, hc


def check_fwd(w, dtype, scale=1.0):
    o, ht, _ = run_fwd(w, scale)
    o_ref, ht_ref = oracle.fwd(**w.tok.f64(), scale=scale, h0=w.h0.astype(np.float64))
    e_o, e_h = rel_max(host(o), o_ref), rel_max(host(ht), ht_ref)
    print(f"  o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < TOL[dtype] and e_h < TOL[dtype]
    return o, ht


def check_bwd(w, dtype, seed, scale=1.0):
    import torch
    from gated_delta_rule_sign_amd import ckda
    B, T, H, DK = w.tok.q.shape
    DV = w.tok.v.shape[-1]
    rng = np.random.default_rng(seed)
    do = I.to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    dht = rng.standard_normal((B, H, DK, DV)).astype(np.float32)
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0)
    _, _, hc = ckda.fwd(**d, scale=scale, h0=h0, want_ckpt=True)
    r = ckda.bwd(**d, h_ckpt=hc, do=dev_tensor(do), scale=scale, h0=h0, dht=dev_tensor(dht))
    torch.cuda.synchronize()
    ref = oracle.bwd(**w.tok.f64(), do=I.widen(do), scale=scale, h0=w.h0.astype(np.float64),
                     dht=dht.astype(np.float64))
    chains = [(b, h) for b in range(B) for h in range(H)]
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        g = host(r[name])
        g = g[bi, :, hi] if g.ndim == 3 else g[bi, :, hi, :]
        e = rel_max(g, ref[name])
        print(f"  {name}: {e:.2e}")
        assert e < TOL[dtype], (name, e)
    e = rel_max(host(r["dh0"]).reshape(B * H, DK, DV), ref["dh0"])
    print(f"  dh0: {e:.2e}")
    assert e < TOL[dtype]


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_forward_gates_at_the_anchor_limit(dtype, DK, DV):
    """Even channels decay by e^-4.9 every token (16-token runs sum to -78.4),
    odd channels keep the workload's gates; signs as drawn."""
    require_gpu()
    banner(f"fwd strong gates {dtype} DK={DK} DV={DV}")
    w = I.make_forward(2, 200, 2, DK, DV, dtype, seed=501, h0_std=0.3)
    w.tok.g[..., 0::2] = -4.9
    check_fwd(w, dtype, scale=0.8)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_backward_gates_at_the_anchor_limit(dtype, DK, DV):
    """Even channels decay by e^-2.45 every token (32-token runs sum to
    -78.4): the backward's own anchor limit."""
    require_gpu()
    banner(f"bwd strong gates {dtype} DK={DK} DV={DV}")
    w = I.make_forward(1, 200, 2, DK, DV, dtype, seed=502, h0_std=0.3)
    w.tok.g[..., 0::2] = -2.45
    check_bwd(w, dtype, seed=503, scale=0.8)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 128), ("bf16", 128, 64)])
def test_beta_zero_only_decays_the_initial_state(dtype, DK, DV):
    require_gpu()
    banner(f"fwd beta=0 {dtype} DK={DK} DV={DV}")
    w = I.make_forward(1, 150, 2, DK, DV, dtype, seed=504, h0_std=0.5)
    w.tok.beta[...] = 0.0
    w.tok.g[...] *= 0.05   # slow decay, so the initial state stays visible over 150 tokens
    check_fwd(w, dtype)
    check_bwd(w, dtype, seed=505)


@pytest.mark.parametrize("dtype,T,DK,DV", [("f32", 256, 32, 64), ("f32", 256, 128, 128), ("bf16", 256, 128, 128),
                                           ("bf16", 1024, 64, 128)])
def test_beta_two_unit_gates_reflections(dtype, T, DK, DV):
    """beta = 2, g = 0 (|alpha| = 1), signs at random: orthogonal transitions
    over T tokens, forward, backward and decode.  Nothing decays, so every
    rounding the chunk records carry stays in the state; a float64 model of
    the bf16 storage gives 1.1e-4 at T = 1024."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner(f"beta=2 g=0 {dtype} T={T} DK={DK} DV={DV}")
    w = I.make_forward(1, T, 2, DK, DV, dtype, seed=506, h0_std=0.3)
    w.tok.beta[...] = 2.0
    w.tok.g[...] = 0.0
    check_fwd(w, dtype)
    check_bwd(w, dtype, seed=507)
    # decode on the same tokens, one step at a time, from the same state
    tok = w.tok
    steps = 40
    st = I.TokenInputs(**{k: np.ascontiguousarray(np.moveaxis(getattr(tok, k)[:, :steps], 1, 0))
                          for k in ("q", "k", "v", "g", "s", "beta")}, dtype=tok.dtype)
    d = tok_to_dev(st)
    state = dev_tensor(w.h0.astype(np.float32))
    sp = torch.ones((1, 2, DK), dtype=torch.int8, device="cuda:0")
    outs = []
    for t in range(steps):
        outs.append(host(ckda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["s"][t],
                                          d["beta"][t], state, sp)))
    torch.cuda.synchronize()
    o_ref, ST, PT = oracle.decode(**st.f64(), state0=w.h0.astype(np.float64))
    assert rel_max(np.stack(outs).reshape(steps, 2, DV), o_ref) < TOL[dtype]
    true_state = (host(sp).astype(np.float64)[..., None] * host(state)).reshape(2, DK, DV)
    assert rel_max(true_state, ST) < TOL[dtype]
    assert np.array_equal(host(sp).reshape(2, DK), PT.astype(np.int8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_query_and_key_rows(dtype):
    require_gpu()
    banner(f"fwd zero q/k rows {dtype}")
    w = I.make_forward(1, 140, 2, 64, 64, dtype, seed=508, h0_std=0.3)
    zq = [0, 17, 63, 64, 100, 139]
    zk = [1, 31, 32, 70, 99]
    w.tok.q[0, zq] = 0
    w.tok.k[0, zk] = 0
    o, _ = check_fwd(w, dtype)
    assert not np.any(host(o)[0, zq])      # a zero query reads exactly zero
    check_bwd(w, dtype, seed=509)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 64, 128)])
def test_segmented_passes_without_decay(dtype, DK, DV):
    """beta = 2, g = 0 over 4,160 tokens (65 chunks) with segments of 16
    chunks forced: five segments, so the scan chains three middle segments
    whose maps P_s are products of orthogonal chunk maps (nothing shrinks),
    forward and backward against the oracle."""
    require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner(f"segments, beta=2 g=0 {dtype} DK={DK} DV={DV}")
    w = I.make_forward(1, 4160, 1, DK, DV, dtype, seed=510, h0_std=0.3)
    w.tok.beta[...] = 2.0
    w.tok.g[...] = 0.0
    ckda.set_segment_chunks(16)
    try:
        check_fwd(w, dtype)
        check_bwd(w, dtype, seed=511)
    finally:
        ckda.set_segment_chunks(0)
