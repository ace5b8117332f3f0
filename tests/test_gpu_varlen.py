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
