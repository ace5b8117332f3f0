"""Packed-document forward on the GPU against the oracle."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128), ("f32", 32, 128)])
def test_varlen_ragged_documents(dtype, DK, DV):
    torch = require_gpu()
    banner(f"varlen ragged {dtype} DK={DK} DV={DV}")
    from gated_delta_rule_sign_amd import ckda
    lens = [0, 1, 63, 64, 65, 130, 0, 200]
    cu = I.cu_from_lengths(lens)
    Tt, H = int(cu[-1]), 2
    rng = np.random.default_rng(5)
    tok = I.draw_tokens(rng, (Tt,), H, DK, DV, dtype)
    h0 = I.draw_state(rng, (len(lens), H, DK, DV), 0.3)
    d = tok_to_dev(tok)
    import torch as T_
    o, ht = ckda.fwd_varlen(**d, cu_seqlens=T_.from_numpy(cu), scale=0.9, h0=dev_tensor(h0))
    torch.cuda.synchronize()
    f = tok.f64()
    o_ref, ht_ref = oracle.varlen(**f, cu_seqlens=cu, scale=0.9, h0=h0.astype(np.float64))
    tol = 1e-4 if dtype == "f32" else 2e-3
    assert rel_max(host(o), o_ref) < tol
    assert rel_max(host(ht), ht_ref) < tol
    # empty documents hand back their initial state untouched
    assert T_.equal(ht[0], dev_tensor(h0)[0]) and T_.equal(ht[6], dev_tensor(h0)[6])


def test_varlen_64k_sampled():
    torch = require_gpu()
    banner("varlen_64k full size, sampled")
    from gated_delta_rule_sign_amd import ckda
    import torch as T_
    w = I.make_workload("varlen_64k")
    d = tok_to_dev(w.tok)
    o, ht = ckda.fwd_varlen(**d, cu_seqlens=T_.from_numpy(w.cu_seqlens), h0=dev_tensor(w.h0))
    torch.cuda.synchronize()
    o = o.cpu().numpy(); ht = ht.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    docs, heads, cols = [0, 5, 15], [0, 9], [2, 40, 77, 127]
    f = w.tok.f64()
    o_ref, ht_ref = oracle.varlen(**f, cu_seqlens=w.cu_seqlens, h0=w.h0.astype(np.float64),
                                  docs=docs, heads=heads, cols=cols)
    cu = w.cu_seqlens
    for n in docs:
        a, b = int(cu[n]), int(cu[n + 1])
        for h in heads:
            e_o = rel_max(o[a:b, h][:, cols].astype(np.float64), o_ref[a:b, h])
            e_h = rel_max(ht[n, h][:, cols].astype(np.float64), ht_ref[n, h])
            assert e_o < 1e-2 and e_h < 1e-2, (n, h, e_o, e_h)


@pytest.mark.parametrize("dtype,DK,DV", [("f32", 64, 64), ("bf16", 128, 128), ("f32", 128, 32)])
def test_varlen_backward_ragged_documents(dtype, DK, DV):
    """ckda_bwd_varlen on ragged documents (empty, 1 token, chunk-boundary
    lengths) against the oracle's backward run on each document alone."""
    torch = require_gpu()
    banner(f"varlen backward ragged {dtype} DK={DK} DV={DV}")
    from gated_delta_rule_sign_amd import ckda
    import torch as T_
    lens = [0, 1, 63, 64, 65, 130, 0, 200]
    cu = I.cu_from_lengths(lens)
    Tt, H, N = int(cu[-1]), 2, len(lens)
    rng = np.random.default_rng(9)
    tok = I.draw_tokens(rng, (Tt,), H, DK, DV, dtype)
    h0 = I.draw_state(rng, (N, H, DK, DV), 0.3)
    do = I.to_storage(rng.standard_normal((Tt, H, DV)), dtype)
    dht = rng.standard_normal((N, H, DK, DV)).astype(np.float32)
    d = tok_to_dev(tok)
    cu_t = T_.from_numpy(cu)
    _, _, hc = ckda.fwd_varlen(**d, cu_seqlens=cu_t, scale=0.7, h0=dev_tensor(h0), want_ckpt=True)
    r = ckda.bwd_varlen(**d, cu_seqlens=cu_t, h_ckpt=hc, do=dev_tensor(do), scale=0.7, h0=dev_tensor(h0),
                        dht=dev_tensor(dht))
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in r.items()}
    f = tok.f64()
    dof = I.widen(do)
    names = ("dq", "dk", "dv", "dg", "dbeta")
    g_all = {k: [] for k in names}
    r_all = {k: [] for k in names}
    dh0_ref = np.zeros((N, H, DK, DV))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:   # an empty document passes dht straight through
            dh0_ref[n] = dht[n]
            continue
        sl = {k: f[k][a:b][None] for k in ("q", "k", "v", "g", "s", "beta")}
        ref = oracle.bwd(**sl, do=dof[a:b][None], scale=0.7, h0=h0[n][None].astype(np.float64),
                         dht=dht[n][None].astype(np.float64))
        for k in names:   # oracle chains are (0, h): [H, len, ...] -> [len, H, ...]
            g_all[k].append(got[k][a:b])
            r_all[k].append(np.moveaxis(ref[k], 0, 1))
        dh0_ref[n] = ref["dh0"]
    design = 1e-4 if dtype == "f32" else 1e-3
    for k in names:
        e = rel_max(np.concatenate(g_all[k]), np.concatenate(r_all[k]))
        print(f"  {k}: {e:.2e}")
        assert e < design, (k, e)
    e = rel_max(got["dh0"], dh0_ref)
    print(f"  dh0: {e:.2e}")
    assert e < design
    assert np.array_equal(got["dh0"][0], dht[0]) and np.array_equal(got["dh0"][6], dht[6])
