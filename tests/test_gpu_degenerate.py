"""Degenerate and extreme inputs of the method on the GPU, against the oracle.

- Deep gates (|alpha| far below 1, the whole of the pages' range [-1, 1]):
  the forward's fast path factors e^{b_r - b_i} through anchors inside each
  half chunk and is used while every 16-token tile's in-tile log-gate prefix
  stays within 96 (log2 units, about 66.5 nat); a chunk beyond that takes
  the exact path, which forms the intra-chunk products entry by entry.  Both
  sides of that boundary are run, on half of the channels, the other half
  keeping ordinary gates, with chunks of both kinds in one call.  The
  backward's chunk-parallel passes use the same anchors, envelope and exact
  path, and are run over the same gates.
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


@pytest.mark.parametrize("dtype,DK,DV,gdeep", [("f32", 64, 64, -4.0), ("bf16", 128, 128, -4.0),
                                              ("f32", 64, 64, -4.9), ("bf16", 128, 128, -4.9),
                                              ("f32", 128, 128, -8.0), ("bf16", 128, 128, -8.0),
                                              ("f32", 64, 128, -40.0), ("bf16", 128, 64, -40.0),
                                              ("f32", 32, 32, -40.0)])
def test_forward_deep_gates(dtype, DK, DV, gdeep):
    """Even channels decay by e^gdeep every token, odd channels keep the
    workload's gates; signs as drawn.  16-token runs of the even channels sum
    to 16 gdeep: -64 (inside the fast path's envelope of about -66.5), -78.4,
    -128 and -640 (beyond it: the exact path)."""
    require_gpu()
    banner(f"fwd deep gates g={gdeep} {dtype} DK={DK} DV={DV}")
    w = I.make_forward(2, 200, 2, DK, DV, dtype, seed=501, h0_std=0.3)
    w.tok.g[..., 0::2] = gdeep
    check_fwd(w, dtype, scale=0.8)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_forward_deep_bursts_inside_chunks(dtype, DK, DV):
    """Tokens 20..27 of every second chunk decay by e^-30 on even channels,
    the rest keeps the workload's gates: pairs across the burst vanish, pairs
    on either side keep O(1) factors between large cumulative log-gates, and
    flagged and unflagged chunks meet in one state pass."""
    require_gpu()
    banner(f"fwd deep bursts {dtype} DK={DK} DV={DV}")
    w = I.make_forward(2, 300, 2, DK, DV, dtype, seed=512, h0_std=0.3)
    for c0 in range(64, 300, 128):
        w.tok.g[:, c0 + 20:c0 + 28, :, 0::2] = -30.0
    check_fwd(w, dtype, scale=0.8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_positive_gates(dtype):
    """g > 0 (|alpha| > 1) lies outside the pages' range; such chunks take
    the exact path, which stays exact while nothing overflows: a few tokens
    with g = +0.4 on some channels."""
    require_gpu()
    banner(f"fwd positive gates {dtype}")
    w = I.make_forward(1, 200, 2, 64, 64, dtype, seed=513, h0_std=0.3)
    w.tok.g[:, 10::37, :, 0::3] = 0.4
    check_fwd(w, dtype, scale=0.8)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_varlen_deep_gates(dtype, DK, DV):
    """Ragged documents, the second and fourth with e^-40 decay on even
    channels (exact path), the others ordinary (fast path)."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner(f"varlen deep gates {dtype} DK={DK} DV={DV}")
    lens = [70, 129, 1, 200, 64]
    cu = I.cu_from_lengths(lens)
    Tt, H = int(cu[-1]), 2
    rng = np.random.default_rng(514)
    tok = I.draw_tokens(rng, (Tt,), H, DK, DV, dtype)
    for n in (1, 3):
        tok.g[cu[n]:cu[n + 1], :, 0::2] = -40.0
    h0 = I.draw_state(rng, (len(lens), H, DK, DV), 0.3)
    d = tok_to_dev(tok)
    o, ht = ckda.fwd_varlen(**d, cu_seqlens=torch.from_numpy(cu), scale=0.9, h0=dev_tensor(h0))
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.varlen(**tok.f64(), cu_seqlens=cu, scale=0.9, h0=h0.astype(np.float64))
    e_o, e_h = rel_max(host(o), o_ref), rel_max(host(ht), ht_ref)
    print(f"  o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < TOL[dtype] and e_h < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_gate_deep(dtype):
    """One gate per (token, head), e^-40 on the first head, ordinary on the
    second."""
    require_gpu()
    banner(f"fwd head gate deep {dtype}")
    w = I.make_forward(1, 200, 2, 64, 64, dtype, seed=515, h0_std=0.3, gate="head")
    w.tok.g[:, :, 0] = -40.0
    o, ht, _ = run_fwd(w, 0.8)
    tok = w.tok.f64()
    DK = w.tok.q.shape[-1]
    tok["g"] = np.repeat(tok["g"][..., None], DK, axis=-1)
    tok["s"] = np.repeat(tok["s"][..., None], DK, axis=-1)
    o_ref, ht_ref = oracle.fwd(**tok, scale=0.8, h0=w.h0.astype(np.float64))
    e_o, e_h = rel_max(host(o), o_ref), rel_max(host(ht), ht_ref)
    print(f"  o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < TOL[dtype] and e_h < TOL[dtype]


@pytest.mark.parametrize("dtype,DK,DV,gdeep", [("f32", 64, 64, -2.45), ("bf16", 128, 128, -2.45),
                                              ("f32", 64, 64, -4.0), ("bf16", 128, 128, -4.0),
                                              ("f32", 64, 64, -4.9), ("bf16", 128, 128, -4.9),
                                              ("f32", 128, 128, -8.0), ("bf16", 128, 128, -8.0),
                                              ("f32", 64, 128, -40.0), ("bf16", 128, 64, -40.0),
                                              ("f32", 32, 32, -40.0)])
def test_backward_deep_gates(dtype, DK, DV, gdeep):
    """The backward over the forward's deep-gate cases: even channels decay by
    e^gdeep every token (16-token runs of -39.2, -64, -78.4, -128, -640),
    odd channels keep the workload's gates; every gradient and dh0 against
    the oracle."""
    require_gpu()
    banner(f"bwd deep gates g={gdeep} {dtype} DK={DK} DV={DV}")
    w = I.make_forward(2, 200, 2, DK, DV, dtype, seed=502, h0_std=0.3)
    w.tok.g[..., 0::2] = gdeep
    check_bwd(w, dtype, seed=503, scale=0.8)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_backward_deep_bursts_inside_chunks(dtype, DK, DV):
    """Tokens 20..27 of every second chunk decay by e^-30 on even channels:
    flagged and unflagged chunks meet in one reverse pass."""
    require_gpu()
    banner(f"bwd deep bursts {dtype} DK={DK} DV={DV}")
    w = I.make_forward(2, 300, 2, DK, DV, dtype, seed=512, h0_std=0.3)
    for c0 in range(64, 300, 128):
        w.tok.g[:, c0 + 20:c0 + 28, :, 0::2] = -30.0
    check_bwd(w, dtype, seed=516, scale=0.8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_positive_gates(dtype):
    """g > 0 on a few tokens and channels (outside the pages' range): the
    exact variants of the backward's chunk passes."""
    require_gpu()
    banner(f"bwd positive gates {dtype}")
    w = I.make_forward(1, 200, 2, 64, 64, dtype, seed=513, h0_std=0.3)
    w.tok.g[:, 10::37, :, 0::3] = 0.4
    check_bwd(w, dtype, seed=517, scale=0.8)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_varlen_backward_deep_gates(dtype, DK, DV):
    """Ragged documents, the second and fourth with e^-40 decay on even
    channels (exact variants), the others ordinary; per document against the
    oracle's backward on that document alone."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    banner(f"varlen backward deep gates {dtype} DK={DK} DV={DV}")
    lens = [70, 129, 1, 200, 64]
    cu = I.cu_from_lengths(lens)
    Tt, H, N = int(cu[-1]), 2, len(lens)
    rng = np.random.default_rng(518)
    tok = I.draw_tokens(rng, (Tt,), H, DK, DV, dtype)
    for n in (1, 3):
        tok.g[cu[n]:cu[n + 1], :, 0::2] = -40.0
    h0 = I.draw_state(rng, (N, H, DK, DV), 0.3)
    do = I.to_storage(rng.standard_normal((Tt, H, DV)), dtype)
    dht = rng.standard_normal((N, H, DK, DV)).astype(np.float32)
    d = tok_to_dev(tok)
    cu_t = torch.from_numpy(cu)
    _, _, hc = ckda.fwd_varlen(**d, cu_seqlens=cu_t, scale=0.9, h0=dev_tensor(h0), want_ckpt=True)
    r = ckda.bwd_varlen(**d, cu_seqlens=cu_t, h_ckpt=hc, do=dev_tensor(do), scale=0.9, h0=dev_tensor(h0),
                        dht=dev_tensor(dht))
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in r.items()}
    f = tok.f64()
    dof = I.widen(do)
    names = ("dq", "dk", "dv", "dg", "dbeta")
    g_all = {k: [] for k in names}
    r_all = {k: [] for k in names}
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = {k: f[k][a:b][None] for k in ("q", "k", "v", "g", "s", "beta")}
        ref = oracle.bwd(**sl, do=dof[a:b][None], scale=0.9, h0=h0[n][None].astype(np.float64),
                         dht=dht[n][None].astype(np.float64))
        for k in names:   # oracle chains are (0, h): [H, len, ...] -> [len, H, ...]
            g_all[k].append(got[k][a:b])
            r_all[k].append(np.moveaxis(ref[k], 0, 1))
        e = rel_max(got["dh0"][n], ref["dh0"])
        assert e < TOL[dtype], ("dh0", n, e)
    for k in names:
        e = rel_max(np.concatenate(g_all[k]), np.concatenate(r_all[k]))
        print(f"  {k}: {e:.2e}")
        assert e < TOL[dtype], (k, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_gate_backward_deep(dtype):
    """One gate per (token, head), e^-40 on the first head, ordinary on the
    second: dg per (token, head) against the oracle's channel-gate gradient
    summed over the channels."""
    import torch
    from gated_delta_rule_sign_amd import ckda
    require_gpu()
    banner(f"bwd head gate deep {dtype}")
    w = I.make_forward(1, 200, 2, 64, 64, dtype, seed=519, h0_std=0.3, gate="head")
    w.tok.g[:, :, 0] = -40.0
    B, T, H, DK = w.tok.q.shape
    DV = w.tok.v.shape[-1]
    rng = np.random.default_rng(520)
    do = I.to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0)
    _, _, hc = ckda.fwd(**d, scale=0.8, h0=h0, want_ckpt=True)
    r = ckda.bwd(**d, h_ckpt=hc, do=dev_tensor(do), scale=0.8, h0=h0)
    torch.cuda.synchronize()
    tok = w.tok.f64()
    tok["g"] = np.repeat(tok["g"][..., None], DK, axis=-1)
    tok["s"] = np.repeat(tok["s"][..., None], DK, axis=-1)
    ref = oracle.bwd(**tok, do=I.widen(do), scale=0.8, h0=w.h0.astype(np.float64))
    bi = [0, 0]; hi = [0, 1]
    for name in ("dq", "dk", "dv", "dbeta"):
        g = host(r[name])
        g = g[bi, :, hi] if g.ndim == 3 else g[bi, :, hi, :]
        e = rel_max(g, ref[name])
        print(f"  {name}: {e:.2e}")
        assert e < TOL[dtype], (name, e)
    e = rel_max(host(r["dg"])[bi, :, hi], ref["dg"].sum(axis=-1))
    print(f"  dg (head): {e:.2e}")
    assert e < TOL[dtype]


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
