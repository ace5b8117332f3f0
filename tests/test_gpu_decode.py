"""Decode step on the GPU against the oracle (single-token recurrence)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu


def run_decode(torch, w, steps, sign0=None):
    from gated_delta_rule_sign_amd import ckda
    tok = w.tok
    N, H, DK, DV = w.h0.shape
    state = dev_tensor(w.h0)
    sp = torch.ones((N, H, DK), dtype=torch.int8, device="cuda:0") if sign0 is None else dev_tensor(sign0)
    d = tok_to_dev(tok)
    outs = []
    for t in range(steps):
        outs.append(ckda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["s"][t], d["beta"][t],
                                     state, sp, scale=0.75))
    torch.cuda.synchronize()
    return np.stack([host(o) for o in outs]), host(state), sp.cpu().numpy()


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 32, 32), ("f32", 64, 128), ("bf16", 128, 128),
                                         ("bf16", 128, 32), ("f32", 32, 64)])
def test_decode_small(dtype, DK, DV):
    torch = require_gpu()
    banner(f"decode small {dtype} DK={DK} DV={DV}")
    N, H, steps = 3, 2, 20
    rng = np.random.default_rng(7)
    state0 = I.draw_state(rng, (N, H, DK, DV), 0.5)
    tok = I.decode_steps(77, 0, steps, N, H, DK, DV, dtype)
    sign0 = np.where(rng.random((N, H, DK)) < 0.5, -1, 1).astype(np.int8)
    w = I.Workload(name="dec", cfg={}, tok=tok, h0=state0)
    o, st, sp = run_decode(torch, w, steps, sign0)
    f = tok.f64()
    o_ref, S_ref, P_ref = oracle.decode(**f, state0=state0.astype(np.float64), sign0=sign0, scale=0.75)
    true_gpu = sp.reshape(N * H, DK, 1).astype(np.float64) * st.reshape(N * H, DK, DV)
    tol = 1e-4 if dtype == "f32" else 1e-2
    assert rel_max(o.reshape(steps, N * H, DV), o_ref) < tol
    assert rel_max(true_gpu, S_ref) < tol
    assert np.array_equal(sp.reshape(N * H, DK), P_ref.astype(np.int8))


def test_decode_b256_shortened():
    """The 256-sequence x 16-head decode workload, first 6 steps, sampled pairs."""
    torch = require_gpu()
    banner("decode_b256 6 steps")
    w = I.make_workload("decode_b256", steps=6)
    o, st, sp = run_decode(torch, w, 6)
    N, H, DK, DV = w.h0.shape
    rng = np.random.default_rng(3)
    pairs = [(int(n), int(h)) for n, h in zip(rng.integers(0, N, 24), rng.integers(0, H, 24))]
    f = w.tok.f64()
    o_ref, S_ref, P_ref = oracle.decode(**f, state0=w.h0.astype(np.float64), scale=0.75, pairs=pairs)
    ni = [p[0] for p in pairs]; hi = [p[1] for p in pairs]
    o_g = o[:, ni, hi, :]
    true_gpu = sp[ni, hi, :, None].astype(np.float64) * st[ni, hi]
    assert rel_max(o_g, o_ref) < 1e-2
    assert rel_max(true_gpu, S_ref) < 1e-2
    assert np.array_equal(sp[ni, hi], P_ref.astype(np.int8))
    # the whole output is finite
    assert np.isfinite(o).all() and np.isfinite(st).all()


def test_decode_b256_bench_configuration():
    """decode_b256 as the benchmark times it: 256 sequences x 16 heads, step
    inputs drawn for 64 steps and used cyclically over 8 + 512 steps, one
    preallocated output, scale 1.  32 sampled (sequence, head) pairs are
    checked against the oracle at three steps and for the final state and
    sign product."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    distinct, total = 64, 8 + 512
    banner(f"decode_b256 {total} steps over {distinct} distinct inputs")
    w = I.make_workload("decode_b256", steps=distinct)
    tok = w.tok
    N, H, DK, DV = w.h0.shape
    d = tok_to_dev(tok)
    state = dev_tensor(w.h0)
    sp = torch.ones((N, H, DK), dtype=torch.int8, device="cuda:0")
    o = torch.empty((N, H, DV), dtype=torch.float32, device="cuda:0")
    checked = (63, 300, total - 1)
    kept = {}
    for t in range(total):
        j = t % distinct
        ckda.decode_step(d["q"][j], d["k"][j], d["v"][j], d["g"][j], d["s"][j], d["beta"][j], state, sp, o=o)
        if t in checked:
            kept[t] = o.clone()
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    ni = rng.integers(0, N, 32)
    hi = rng.integers(0, H, 32)
    cyc = np.arange(total) % distinct

    def pick(x):   # [distinct, N, H, ...] -> [total, 32, 1, ...] for the sampled pairs
        return np.ascontiguousarray(np.asarray(x)[:, ni, hi][cyc][:, :, None])

    o_ref, S_ref, P_ref = oracle.decode(q=I.widen(pick(tok.q)), k=I.widen(pick(tok.k)), v=I.widen(pick(tok.v)),
                                        g=pick(tok.g).astype(np.float64), s=pick(tok.s).astype(np.float64),
                                        beta=pick(tok.beta).astype(np.float64),
                                        state0=w.h0[ni, hi][:, None].astype(np.float64))
    for t in checked:
        e = rel_max(host(kept[t])[ni, hi], o_ref[t])
        print(f"  o at step {t}: {e:.2e}")
        assert e < 1e-3
    true_gpu = host(sp)[ni, hi][:, :, None].astype(np.float64) * host(state)[ni, hi]
    e = rel_max(true_gpu, S_ref)
    print(f"  final state: {e:.2e}")
    assert e < 1e-3
    assert np.array_equal(host(sp)[ni, hi], P_ref.astype(np.int8))
    assert np.isfinite(host(state)).all()
