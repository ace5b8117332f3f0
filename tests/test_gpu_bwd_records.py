"""The backward reading the forward's own chunk records (ckda_bwd_with_records,
ckda_bwd_varlen_with_records): the reverse pass stages the forward record's
W, Qh, KbT and M transposed instead of reverse records of its own.  Checked
against the oracle at the contract tolerances and against the backward that
writes its own reverse records (the two record kinds round the same
quantities in different orders, so they agree to rounding, not bitwise):
several head sizes and both dtypes, ragged tails, h0 and dht, deep gates
whose chunks take the exact path, varlen documents and the segmented reverse
pass."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu

# against the oracle: the contract bounds, and for these small cases the
# backward's design bounds (as in test_gpu_bwd.py)
TOL = {"f32": 1e-4, "bf16": 1e-2}
DESIGN = {"f32": 1e-4, "bf16": 1e-3}
# with records against without: the forward record's KbT is formed through
# the anchors, the reverse record's KB directly, so the two differ by fp32
# rounding (bf16 inputs: in hi/lo pairs, about 2^-16 of each element), and
# the reverse recurrence carries that into every gradient
AGREE = {"f32": 1e-5, "bf16": 1e-3}
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def run_both(w, do, dht, scale, dtype):
    import torch
    from gated_delta_rule_sign_amd import ckda
    B, T, H, DK = w.tok.q.shape
    DV = w.tok.v.shape[-1]
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0)
    ws = torch.empty(ckda.fwd_workspace_bytes(B, T, H, DK, DV, d["q"].dtype), dtype=torch.uint8, device="cuda:0")
    _, _, hc = ckda.fwd(**d, scale=scale, h0=h0, want_ckpt=True, workspace=ws)
    kw = dict(h_ckpt=hc, do=dev_tensor(do), scale=scale, h0=h0, dht=dev_tensor(dht))
    r_rec = ckda.bwd(**d, **kw, fwd_workspace=ws)
    r_own = ckda.bwd(**d, **kw)
    torch.cuda.synchronize()
    return r_rec, r_own


def check(w, do, dht, scale, dtype, r_rec, r_own):
    B, T, H, DK = w.tok.q.shape
    DV = w.tok.v.shape[-1]
    for name in NAMES:
        e = rel_max(host(r_rec[name]), host(r_own[name]))
        print(f"  {name} records vs own: {e:.2e}")
        assert e < AGREE[dtype], (name, e)
    ref = oracle.bwd(**w.tok.f64(), do=I.widen(do), scale=scale, h0=w.h0.astype(np.float64),
                     dht=dht.astype(np.float64))
    chains = [(b, h) for b in range(B) for h in range(H)]
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    for name in NAMES[:-1]:
        g = host(r_rec[name])
        g = g[bi, :, hi] if g.ndim == 3 else g[bi, :, hi, :]
        e = rel_max(g, ref[name])
        print(f"  {name} vs oracle: {e:.2e}")
        assert e < DESIGN[dtype], (name, e)
    assert rel_max(host(r_rec["dh0"]).reshape(B * H, DK, DV), ref["dh0"]) < DESIGN[dtype]


@pytest.mark.parametrize("dtype,B,T,H,DK,DV", [("f32", 1, 130, 2, 64, 64), ("bf16", 2, 200, 2, 128, 128),
                                               ("f32", 2, 64, 1, 32, 128), ("bf16", 1, 96, 2, 128, 32),
                                               ("bf16", 2, 128, 2, 64, 64), ("f32", 1, 1, 1, 32, 32)])
def test_with_records_small(dtype, B, T, H, DK, DV):
    require_gpu()
    banner(f"bwd with forward records {dtype} B={B} T={T} H={H} DK={DK} DV={DV}")
    w = I.make_forward(B, T, H, DK, DV, dtype, seed=61 + T, h0_std=0.3)
    rng = np.random.default_rng(T + 3)
    do = I.to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    dht = rng.standard_normal((B, H, DK, DV)).astype(np.float32)
    r_rec, r_own = run_both(w, do, dht, 0.7, dtype)
    check(w, do, dht, 0.7, dtype, r_rec, r_own)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128)])
def test_with_records_deep_gates(dtype, DK, DV):
    """Even channels at e^-40 per token: every chunk leaves the anchors'
    envelope, so the forward's records come from its exact path and their
    flags send the gradient phases to theirs."""
    require_gpu()
    banner(f"bwd with forward records, deep gates {dtype} DK={DK} DV={DV}")
    w = I.make_forward(2, 200, 2, DK, DV, dtype, seed=502, h0_std=0.3)
    w.tok.g[..., 0::2] = -40.0
    rng = np.random.default_rng(9)
    do = I.to_storage(rng.standard_normal((2, 200, 2, DV)), dtype)
    dht = rng.standard_normal((2, 2, DK, DV)).astype(np.float32)
    r_rec, r_own = run_both(w, do, dht, 0.8, dtype)
    check(w, do, dht, 0.8, dtype, r_rec, r_own)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_with_records(dtype):
    """Ragged documents (an empty one included) with per-document h0 and dht,
    against the oracle's backward run on each document alone."""
    import torch
    require_gpu()
    from gated_delta_rule_sign_amd import ckda
    lens = [5, 0, 64, 130, 1, 77]
    cu = I.cu_from_lengths(lens)
    Tt, N, H, DK, DV = int(cu[-1]), len(lens), 2, 64, 64
    banner(f"bwd varlen with forward records {dtype} T={Tt} N={N}")
    rng = np.random.default_rng(5)
    tok = I.draw_tokens(rng, (Tt,), H, DK, DV, dtype)
    h0 = I.draw_state(rng, (N, H, DK, DV), 0.3)
    do = I.to_storage(rng.standard_normal((Tt, H, DV)), dtype)
    dht = rng.standard_normal((N, H, DK, DV)).astype(np.float32)
    d = tok_to_dev(tok)
    cut = torch.from_numpy(np.asarray(cu, np.int32))
    ws = torch.empty(ckda.fwd_varlen_workspace_bytes(N, Tt, H, DK, DV, d["q"].dtype), dtype=torch.uint8,
                     device="cuda:0")
    _, _, hc = ckda.fwd_varlen(**d, cu_seqlens=cut, scale=0.7, h0=dev_tensor(h0), want_ckpt=True, workspace=ws)
    kw = dict(cu_seqlens=cut, h_ckpt=hc, do=dev_tensor(do), scale=0.7, h0=dev_tensor(h0), dht=dev_tensor(dht))
    r_rec = ckda.bwd_varlen(**d, **kw, fwd_workspace=ws)
    r_own = ckda.bwd_varlen(**d, **kw)
    torch.cuda.synchronize()
    for name in NAMES:
        e = rel_max(host(r_rec[name]), host(r_own[name]))
        print(f"  {name} records vs own: {e:.2e}")
        assert e < AGREE[dtype], (name, e)
    got = {k: host(v) for k, v in r_rec.items()}
    f = tok.f64()
    dof = I.widen(do)
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:   # an empty document passes dht straight through
            assert np.array_equal(got["dh0"][n], dht[n])
            continue
        sl = {k: f[k][a:b][None] for k in ("q", "k", "v", "g", "s", "beta")}
        ref = oracle.bwd(**sl, do=dof[a:b][None], scale=0.7, h0=h0[n][None].astype(np.float64),
                         dht=dht[n][None].astype(np.float64))
        for k in ("dq", "dk", "dv", "dg", "dbeta"):   # oracle chains (0, h): [H, len, ...] -> [len, H, ...]
            e = rel_max(got[k][a:b], np.moveaxis(ref[k], 0, 1))
            assert e < DESIGN[dtype], (n, k, e)
        assert rel_max(got["dh0"][n], ref["dh0"].reshape(H, DK, DV)) < DESIGN[dtype]


def test_segmented_reverse_pass_with_records():
    """Forced segments of 16 chunks over a long-memory chain (the maps of the
    middle segments do not vanish), fed by the forward's records."""
    import torch
    require_gpu()
    from gated_delta_rule_sign_amd import ckda
    B, T, H, DK, DV = 2, 3300, 2, 128, 128
    banner(f"bwd with forward records, segmented reverse pass B={B} T={T}")
    w = I.make_forward(B, T, H, DK, DV, "bf16", seed=53 + T, h0_std=0.3)
    w.tok.g *= np.float32(1e-3)
    w.tok.beta *= np.float32(0.05)
    rng = np.random.default_rng(T + 7)
    do = I.to_storage(rng.standard_normal((B, T, H, DV)), "bf16")
    dht = rng.standard_normal((B, H, DK, DV)).astype(np.float32)
    try:
        ckda.set_segment_chunks(16)
        r_rec, r_own = run_both(w, do, dht, 0.8, "bf16")
    finally:
        ckda.set_segment_chunks(0)
    for name in NAMES:
        e = rel_max(host(r_rec[name]), host(r_own[name]))
        print(f"  {name} records vs own: {e:.2e}")
        assert e < AGREE["bf16"], (name, e)


@pytest.mark.parametrize("option", ["head_gate", "qk_norm", "gate_map"])
def test_with_records_and_options(option):
    """The forward's records under each option (one gate per head, q and k
    normalised in the path, the gate map on pre-activations) feed the same
    gradients as the backward's own reverse records; those are held to the
    oracle by the options' own tests."""
    import torch
    require_gpu()
    from gated_delta_rule_sign_amd import ckda
    B, T, H, DK, DV, dtype = 2, 150, 2, 128, 64, "bf16"
    banner(f"bwd with forward records, {option}")
    rng = np.random.default_rng(123)
    tok = I.draw_tokens(rng, (B, T), H, DK, DV, dtype, gate="head" if option == "head_gate" else "channel",
                        qk="raw" if option == "qk_norm" else "unit")
    d = tok_to_dev(tok)
    kw = {}
    if option == "qk_norm":
        kw["qk_norm"] = True
    if option == "gate_map":
        x, y = I.draw_gate_preacts(rng, (B, T, H, DK), (B, T, H))
        d.update(g=dev_tensor(x), s=None, beta=dev_tensor(y))
        kw["gate_map"] = True
    h0 = dev_tensor(I.draw_state(rng, (B, H, DK, DV), 0.3))
    do = dev_tensor(I.to_storage(rng.standard_normal((B, T, H, DV)), dtype))
    dht = dev_tensor(rng.standard_normal((B, H, DK, DV)).astype(np.float32))
    ws = torch.empty(ckda.fwd_workspace_bytes(B, T, H, DK, DV, d["q"].dtype), dtype=torch.uint8, device="cuda:0")
    _, _, hc = ckda.fwd(**d, scale=0.9, h0=h0, want_ckpt=True, workspace=ws, **kw)
    args = dict(h_ckpt=hc, do=do, scale=0.9, h0=h0, dht=dht, **kw)
    r_rec = ckda.bwd(**d, **args, fwd_workspace=ws)
    r_own = ckda.bwd(**d, **args)
    torch.cuda.synchronize()
    for name in NAMES:
        e = rel_max(host(r_rec[name]), host(r_own[name]))
        print(f"  {name} records vs own: {e:.2e}")
        assert e < AGREE[dtype], (name, e)
