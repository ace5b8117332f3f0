"""ckda_fwd_chunked_noalloc (the forward that allocates nothing: its chunk
records live in the library's fixed device scratch) against ckda_fwd_chunked
with a caller workspace, through the C ABI: two calls in a row, the second
smaller and with deep gates on half of the channels (the exact path reads its
flags from the same scratch), then a size beyond the scratch."""
import numpy as np
import pytest

from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu, tok_to_dev

pytestmark = pytest.mark.gpu


def _pair(w):
    import torch
    from gated_delta_rule_sign_amd import ckda
    d = tok_to_dev(w.tok)
    B, T, H, DK = w.tok.q.shape
    DV = w.tok.v.shape[-1]
    h0 = dev_tensor(w.h0)
    NT = (T + 63) // 64
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device="cuda:0")
    ht = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda:0")
    hc = torch.empty((B, H, NT, DK, DV), dtype=torch.float32, device="cuda:0")
    ckda.fwd_noalloc(**d, o=o, ht=ht, h0=h0, h_ckpt=hc, scale=0.8)
    try:
        ckda.set_segment_chunks(-1)      # the no-allocation call keeps whole chains
        o_ref, ht_ref, hc_ref = ckda.fwd(**d, h0=h0, want_ckpt=True, scale=0.8)
    finally:
        ckda.set_segment_chunks(0)
    torch.cuda.synchronize()
    return (o, ht, hc), (o_ref, ht_ref, hc_ref)


def test_noalloc_matches_the_workspace_forward():
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    cases = [
        ("bf16, B=2 T=1000 H=8 d=128", I.make_forward(2, 1000, 8, 128, 128, "bf16", seed=901, h0_std=0.1), None),
        ("f32, B=1 T=300 H=3 d=64, deep gates", I.make_forward(1, 300, 3, 64, 64, "f32", seed=902, h0_std=0.3),
         -40.0),
    ]
    for name, w, deep in cases:
        banner(f"noalloc forward {name}")
        if deep is not None:
            w.tok.g[..., 0::2] = deep
        got, ref = _pair(w)
        tol = 1e-4 if w.tok.dtype == "f32" else 1e-2
        for a, b, what in zip(got, ref, ("o", "ht", "h_ckpt")):
            e = rel_max(host(a), host(b))
            print(f"  {what}: max|diff|/rms {e:.2e}, bitwise {torch.equal(a, b)}")
            assert e <= tol and torch.equal(a, b), what
    # beyond the scratch: refused on the host, nothing enqueued
    banner("noalloc forward beyond the scratch")
    w = I.make_forward(1, 64 * 40, 32, 128, 128, "bf16", seed=903)   # 1,280 chunk-heads
    d = tok_to_dev(w.tok)
    o = torch.zeros((1, 64 * 40, 32, 128), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ckda.CkdaError, match="scratch"):
        ckda.fwd_noalloc(**d, o=o)
    assert not torch.any(o)
