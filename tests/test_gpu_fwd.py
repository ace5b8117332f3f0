"""Chunked forward on the GPU against the oracle, plus properties that hold
bitwise (sign gauge, determinism, chunk-aligned split calls)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu

# contract tolerances (max|diff| / RMS of the oracle): fp32 inputs 1e-4,
# bf16 inputs 1e-2.  For bf16 inputs the chunk records keep W, Qh, KbT and M
# as hi/lo bf16 pairs; a float64 rounding model of that storage gives 1.1e-4
# at T = 4096 (measured: 1.0e-4 .. 1.4e-4), so small cases are also held to a
# tighter design bound to catch regressions early.
TOL = {"f32": 1e-4, "bf16": 1e-2}
DESIGN = {"f32": 1e-4, "bf16": 5e-4}


def gpu_fwd(w, scale=1.0, want_ckpt=False):
    from gated_delta_rule_sign_amd import ckda
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0) if w.h0 is not None else None
    o, ht, hc = ckda.fwd(**d, scale=scale, h0=h0, want_ckpt=want_ckpt)
    import torch
    torch.cuda.synchronize()
    return o, ht, hc


def test_tiny_fp32_workload():
    require_gpu()
    banner("fwd tiny_fp32")
    w = I.make_workload("tiny_fp32")
    o, ht, _ = gpu_fwd(w)
    o_ref, ht_ref = oracle.fwd(**w.tok.f64())
    assert rel_max(host(o), o_ref) < TOL["f32"]
    assert rel_max(host(ht), ht_ref) < TOL["f32"]


CASES = [
    ("f32", 1, 200, 2, 64, 64),
    ("bf16", 2, 130, 2, 128, 128),
    ("f32", 1, 64, 1, 128, 32),
    ("bf16", 1, 1, 3, 32, 128),
    ("f32", 2, 127, 1, 32, 64),
    ("bf16", 1, 333, 2, 64, 128),
    ("f32", 1, 96, 2, 128, 128),
    ("bf16", 2, 200, 2, 32, 32),
    ("bf16", 1, 150, 2, 64, 32),
    ("bf16", 1, 140, 1, 128, 32),
]


@pytest.mark.parametrize("dtype,B,T,H,DK,DV", CASES)
def test_small_shapes_with_state_and_scale(dtype, B, T, H, DK, DV):
    require_gpu()
    banner(f"fwd {dtype} B={B} T={T} H={H} DK={DK} DV={DV}")
    w = I.make_forward(B, T, H, DK, DV, dtype, seed=11 + T, h0_std=0.3)
    o, ht, _ = gpu_fwd(w, scale=0.6)
    f = w.tok.f64()
    o_ref, ht_ref = oracle.fwd(**f, scale=0.6, h0=w.h0.astype(np.float64))
    e_o, e_h = rel_max(host(o), o_ref), rel_max(host(ht), ht_ref)
    print(f"  max|diff|/rms: o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < DESIGN[dtype] and e_h < DESIGN[dtype]


def test_empty_sequence_returns_initial_state():
    torch = require_gpu()
    banner("fwd T=0")
    from gated_delta_rule_sign_amd import ckda
    w = I.make_forward(2, 1, 2, 64, 64, "bf16", seed=3, h0_std=0.5)
    d = {k: v[:, :0].contiguous() for k, v in tok_to_dev(w.tok).items()}
    h0 = dev_tensor(w.h0)
    o, ht, _ = ckda.fwd(**d, h0=h0)
    torch.cuda.synchronize()
    assert o.shape[1] == 0
    assert torch.equal(ht, h0)


def test_checkpoints_are_chunk_start_states():
    require_gpu()
    banner("fwd checkpoints")
    w = I.make_forward(1, 200, 2, 64, 64, "f32", seed=4, h0_std=0.2)
    _, _, hc = gpu_fwd(w, want_ckpt=True)
    hc = host(hc)                                   # [B,H,NT,DK,DV]
    f = w.tok.f64()
    for j in range(hc.shape[2]):
        if j == 0:
            ref = w.h0.astype(np.float64)
        else:
            sub = {k: v[:, :64 * j] for k, v in f.items()}
            _, ref = oracle.fwd(**sub, h0=w.h0.astype(np.float64))
        assert rel_max(hc[:, :, j], ref) < TOL["f32"]


def _gauge_pair(w, sig):
    """Inputs relabelled by key-channel signs sig [B, T+1, H, DK] (sig[:, 0] is
    sigma_{-1}): q, k flipped by sigma_t, the gate sign by sigma_t sigma_{t-1},
    the initial state rows by sigma_{-1}."""
    if w.tok.dtype == "bf16":
        flip = lambda bits, sg: bits ^ np.where(sg < 0, np.uint16(0x8000), np.uint16(0)).astype(np.uint16)
    else:
        flip = lambda x, sg: (x * sg).astype(np.float32)     # exact: a sign change
    tok2 = I.TokenInputs(q=flip(w.tok.q, sig[:, 1:]), k=flip(w.tok.k, sig[:, 1:]), v=w.tok.v, g=w.tok.g,
                         s=(sig[:, 1:] * sig[:, :-1] * w.tok.s).astype(np.int8), beta=w.tok.beta,
                         dtype=w.tok.dtype)
    h02 = (sig[:, 0][..., None] * w.h0).astype(np.float32)
    return I.Workload("g", {}, tok2, h0=h02)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sign_gauge_invariance(dtype):
    """The output does not depend on how the +-1 part of the gate is labelled:
    relabelling by any sigma_t leaves o unchanged and flips ht by
    sigma_{T-1}.  Inside chunk c the relabelled run sees kf, qf, W and Qh with
    the channels of sigma_{c0-1} negated (c0 the chunk's first token), the
    chunk-start state rows negated the same way and KbT, d rows negated by
    sigma at the chunk's last token, so in exact IEEE arithmetic every product
    and sum is the old one or its negation.
    - sigma = +1 at every chunk's last token: the kernels see identical
      operands, bitwise identical results (both dtypes).
    - arbitrary sigma with fp32 inputs (fp32 matrix cores): bitwise.
    - arbitrary sigma with bf16 inputs: equal to the last bits only.  The bf16
      matrix-core product v_mfma_f32_16x16x32_bf16 is not sign-symmetric in its
      last bit: on random operands, (-A) B + (-C) differs from -(A B + C) in
      143 of 1,048,576 outputs on MI355X, while v_mfma_f32_16x16x4_f32 matches
      in all of them."""
    torch = require_gpu()
    banner(f"fwd gauge {dtype}")
    DK = 128 if dtype == "bf16" else 64
    w = I.make_forward(2, 190, 2, DK, DK, dtype, seed=8, h0_std=0.2)
    rng = np.random.default_rng(1)
    B, T, H, DK = w.tok.q.shape
    sig = np.where(rng.random((B, T + 1, H, DK)) < 0.5, -1, 1).astype(np.int8)
    o1, ht1, _ = gpu_fwd(w)
    # (a) +1 at t = -1 and at every chunk's last token: bitwise
    sig_a = sig.copy()
    sig_a[:, 0] = 1
    sig_a[:, 64::64] = 1          # index t+1 = 64, 128, ... is token 63, 127, ...
    sig_a[:, -1] = 1
    o2, ht2, _ = gpu_fwd(_gauge_pair(w, sig_a))
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    # (b) arbitrary sigma
    o3, ht3, _ = gpu_fwd(_gauge_pair(w, sig))
    sT = dev_tensor(sig[:, -1][..., None].astype(np.float32))
    if dtype == "f32":
        assert torch.equal(o3, o1) and torch.equal(ht3, sT * ht1)
    else:
        assert rel_max(host(o3), host(o1)) < 1e-5
        assert rel_max(host(ht3), host(sT * ht1)) < 1e-5


def test_run_to_run_determinism():
    torch = require_gpu()
    banner("fwd determinism")
    w = I.make_forward(2, 300, 4, 128, 128, "bf16", seed=9)
    o1, ht1, _ = gpu_fwd(w)
    o2, ht2, _ = gpu_fwd(w)
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)


def test_split_call_composition():
    torch = require_gpu()
    banner("fwd split calls")
    from gated_delta_rule_sign_amd import ckda
    w = I.make_forward(1, 320, 2, 64, 128, "bf16", seed=12, h0_std=0.1)
    d = tok_to_dev(w.tok)
    h0 = dev_tensor(w.h0)
    o, ht, _ = ckda.fwd(**d, h0=h0)
    for cut, exact in ((128, True), (100, False)):
        a = {k: v[:, :cut].contiguous() for k, v in d.items()}
        b = {k: v[:, cut:].contiguous() for k, v in d.items()}
        oa, hta, _ = ckda.fwd(**a, h0=h0)
        ob, htb, _ = ckda.fwd(**b, h0=hta)
        torch.cuda.synchronize()
        oc = torch.cat([oa, ob], dim=1)
        if exact:   # chunk-aligned cut: identical chunking, identical arithmetic
            assert torch.equal(oc, o) and torch.equal(htb, ht)
        else:       # other chunk boundaries: both runs within the design bound of the oracle
            o_ref, ht_ref = oracle.fwd(**w.tok.f64(), h0=w.h0.astype(np.float64))
            assert rel_max(host(oc), o_ref) < DESIGN["bf16"] and rel_max(host(htb), ht_ref) < DESIGN["bf16"]
            assert rel_max(host(o), o_ref) < DESIGN["bf16"] and rel_max(host(ht), ht_ref) < DESIGN["bf16"]


def test_layer_workload_sampled():
    """B=8, T=4096, H=16, d=128 bf16 (one mixer layer of the 1.36B model):
    the whole output on the GPU, sampled chains and value columns against
    the oracle (value columns evolve independently, so a column subset of the
    oracle is exact for those columns)."""
    torch = require_gpu()
    banner("fwd layer_bf16 full size, sampled")
    w = I.make_workload("layer_bf16")
    o, ht, _ = gpu_fwd(w)
    o = o.cpu().numpy(); ht = ht.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    chains = [(0, 0), (3, 7), (5, 12), (7, 15)]
    cols = [0, 17, 38, 63, 64, 85, 110, 127]
    f = w.tok.f64()
    o_ref, ht_ref = oracle.fwd(**f, chains=chains, cols=cols)
    bi = [c[0] for c in chains]; hi = [c[1] for c in chains]
    o_g = o[bi, :, hi, :][:, :, cols].astype(np.float64)
    ht_g = ht[bi, hi][:, :, cols].astype(np.float64)
    e_o, e_h = rel_max(o_g, o_ref), rel_max(ht_g, ht_ref)
    print(f"  layer_bf16 max|diff|/rms: o {e_o:.2e}  ht {e_h:.2e}")
    assert e_o < TOL["bf16"] and e_h < TOL["bf16"]
