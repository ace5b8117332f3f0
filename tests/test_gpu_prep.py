"""Gate / sign-fold prep kernel against a plain restatement of its
definition (chunk-local fp32 running sum of g, running product of s)."""
import numpy as np
import pytest

from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,T,DK", [("f32", 256, 32), ("bf16", 200, 128), ("bf16", 65, 64)])
def test_chunk_prep(dtype, T, DK):
    torch = require_gpu()
    banner(f"prep {dtype} T={T} DK={DK}")
    from gated_delta_rule_sign_amd import ckda
    w = I.make_forward(2, T, 3, DK, DK, dtype, seed=5)
    tok = w.tok
    b, p, qf, kf = ckda.chunk_prep(dev_tensor(tok.q), dev_tensor(tok.k), dev_tensor(tok.g), dev_tensor(tok.s))
    torch.cuda.synchronize()
    b = b.cpu().numpy(); p = p.cpu().numpy()
    qf = qf.float().cpu().numpy(); kf = kf.float().cpu().numpy()
    q = I.widen(tok.q); k = I.widen(tok.k)
    for c0 in range(0, T, 64):
        sl = slice(c0, min(T, c0 + 64))
        ref_b = np.cumsum(tok.g[:, sl], axis=1, dtype=np.float32)     # sequential fp32 sum
        ref_p = np.cumprod(tok.s[:, sl].astype(np.int32), axis=1)
        assert np.array_equal(b[:, sl], ref_b)
        assert np.array_equal(p[:, sl], ref_p)
        assert np.array_equal(qf[:, sl], ref_p * q[:, sl])
        assert np.array_equal(kf[:, sl], ref_p * k[:, sl])
