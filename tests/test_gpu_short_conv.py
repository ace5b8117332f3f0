"""The optional short convolution (width 4, depthwise, causal) on the GPU
against the oracle: sequences and documents with ragged lengths across the
kernels' 64-token runs, carried windows, SiLU on and off, the backward
(dx, dw, the window's gradient), decode steps continuing a prefill, and the
full layer shapes on sampled channels (channels are independent)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_sign_amd import inputs as I
from tests.gpu_utils import banner, dev_tensor, host, rel_max, require_gpu

pytestmark = pytest.mark.gpu

# fp32 inputs: four fused multiply-adds and, with SiLU, the hardware exp2 and
# a division per element, against float64: a few ulp.  bf16 inputs: the same,
# then one rounding of y to bf16: half an ulp (at most 2^-8 relative, at the
# bottom of a binade), or one ulp where the fp32 error crosses a rounding
# boundary, so y is held elementwise to 2^-7 |y_ref|.
TOL_F32 = 2e-6
BF16_REL = 2.0 ** -7


def check_y(y, ref, dtype):
    if dtype == "f32":
        e = rel_max(y, ref)
        assert e < TOL_F32, e
        return e
    rms = float(np.sqrt(np.mean(ref * ref)))
    bad = np.abs(y - ref) > BF16_REL * np.abs(ref) + 1e-6 * rms
    assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(y - ref))))
    return rel_max(y, ref)


def run_fwd(x, w, s0, cu=None, silu=False):
    from gated_delta_rule_sign_amd import ckda
    import torch
    cut = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32))
    y, st = ckda.short_conv(dev_tensor(x), dev_tensor(w), cu_seqlens=cut,
                            state0=None if s0 is None else dev_tensor(s0), silu=silu, want_state=True)
    torch.cuda.synchronize()
    return y, st


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("B,T,C,state", [(2, 150, 64, True), (3, 64, 2048, False), (1, 1, 32, True),
                                         (2, 2, 1032, True), (4, 333, 1024, False)])
def test_sequences(dtype, silu, B, T, C, state):
    require_gpu()
    banner(f"short conv fwd {dtype} silu={silu} B={B} T={T} C={C} state={state}")
    x, w, s0, _ = I.draw_conv(100 + T + C, (B, T, C), C, B, dtype, with_state=state)
    y, st = run_fwd(x, w, s0, silu=silu)
    y_ref, st_ref = oracle.short_conv(I.widen(x), w, state0=None if s0 is None else I.widen(s0), silu=silu)
    e = check_y(host(y), y_ref, dtype)
    print(f"  y max|diff|/rms {e:.2e}")
    # the outgoing window is a copy of inputs: exact
    assert np.array_equal(host(st), st_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_documents(dtype):
    """Ragged documents, empty ones included, across 64-token runs: each gets
    its own window (or zero history) and hands on its last three inputs."""
    require_gpu()
    lens = [0, 1, 2, 3, 63, 64, 65, 130, 0, 7, 200]
    cu = I.cu_from_lengths(lens)
    T, C, N = int(cu[-1]), 256, len(lens)
    banner(f"short conv documents {dtype} T={T} N={N}")
    x, w, s0, _ = I.draw_conv(7, (T, C), C, N, dtype)
    for silu in (False, True):
        y, st = run_fwd(x, w, s0, cu=cu, silu=silu)
        y_ref, st_ref = oracle.short_conv(I.widen(x), w, cu_seqlens=cu, state0=I.widen(s0), silu=silu)
        check_y(host(y), y_ref, dtype)
        assert np.array_equal(host(st), st_ref)


def test_window_in_place_and_decode_steps_continue_a_prefill():
    """state_out may be state0 itself; decode steps from the outgoing window
    give the same bits as one call over the whole sequence."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    B, T, C = 3, 100, 512
    banner(f"short conv prefill + decode B={B} T={T} C={C}")
    for dtype in ("f32", "bf16"):
        x, w, s0, _ = I.draw_conv(11, (B, T, C), C, B, dtype)
        xd, wd = dev_tensor(x), dev_tensor(w)
        y_all, st_all = ckda.short_conv(xd, wd, state0=dev_tensor(s0), silu=True, want_state=True)
        win = dev_tensor(s0)
        y_pre, _ = ckda.short_conv(xd[:, :90].contiguous(), wd, state0=win, silu=True, state_out=win)
        ys = [ckda.short_conv_step(xd[:, t].contiguous(), wd, win, silu=True) for t in range(90, T)]
        torch.cuda.synchronize()
        assert torch.equal(y_pre, y_all[:, :90])
        assert torch.equal(torch.stack(ys, dim=1), y_all[:, 90:])
        assert torch.equal(win, st_all)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("silu", [False, True])
def test_backward(dtype, silu):
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    lens = [5, 0, 64, 1, 190, 2, 70]
    cu = I.cu_from_lengths(lens)
    T, C, N = int(cu[-1]), 1024 + 64, len(lens)
    banner(f"short conv bwd {dtype} silu={silu} T={T} C={C}")
    x, w, s0, dy = I.draw_conv(21, (T, C), C, N, dtype)
    cut = torch.from_numpy(np.asarray(cu, np.int32))
    r = ckda.short_conv_bwd(dev_tensor(x), dev_tensor(w), dev_tensor(dy), cu_seqlens=cut, state0=dev_tensor(s0),
                            silu=silu, want_dstate0=True)
    r2 = ckda.short_conv_bwd(dev_tensor(x), dev_tensor(w), dev_tensor(dy), cu_seqlens=cut, state0=dev_tensor(s0),
                             silu=silu, want_dstate0=True)
    torch.cuda.synchronize()
    dx_ref, dw_ref, ds_ref = oracle.short_conv_bwd(I.widen(x), w, dy, cu_seqlens=cu, state0=I.widen(s0), silu=silu)
    # dx, dstate0: at most four products per element; dw: a sum over the
    # tokens of each channel in fp32
    e_dx, e_ds, e_dw = rel_max(host(r["dx"]), dx_ref), rel_max(host(r["dstate0"]), ds_ref), rel_max(host(r["dw"]), dw_ref)
    print(f"  dx {e_dx:.2e} dstate0 {e_ds:.2e} dw {e_dw:.2e}")
    assert e_dx < 2e-6 and e_ds < 2e-6 and e_dw < 2e-5
    for k in ("dx", "dw", "dstate0"):   # fixed summation order: the same bits every call
        assert torch.equal(r[k], r2[k]), k


def test_backward_equal_sequences_without_window():
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    B, T, C = 2, 129, 128
    banner(f"short conv bwd equal sequences B={B} T={T} C={C}")
    x, w, _, dy = I.draw_conv(31, (B, T, C), C, B, "bf16", with_state=False)
    r = ckda.short_conv_bwd(dev_tensor(x), dev_tensor(w), dev_tensor(dy), silu=True)
    torch.cuda.synchronize()
    dx_ref, dw_ref, _ = oracle.short_conv_bwd(I.widen(x), w, dy, silu=True)
    assert r["dstate0"] is None
    assert rel_max(host(r["dx"]), dx_ref) < 2e-6
    assert rel_max(host(r["dw"]), dw_ref) < 2e-5


def test_layer_shapes_sampled_channels():
    """q of the layer workload's shapes (B=8, T=4096, 16 heads x 128 = 2048
    channels, bf16) with SiLU, forward and backward, checked on 24 channels
    (every channel is independent of the others)."""
    torch = require_gpu()
    from gated_delta_rule_sign_amd import ckda
    B, T, C = 8, 4096, 2048
    banner(f"short conv layer shapes B={B} T={T} C={C}")
    x, w, _, dy = I.draw_conv(41, (B, T, C), C, B, "bf16", with_state=False)
    xd = dev_tensor(x)
    y, _ = ckda.short_conv(xd, dev_tensor(w), silu=True)
    r = ckda.short_conv_bwd(xd, dev_tensor(w), dev_tensor(dy), silu=True)
    torch.cuda.synchronize()
    cols = np.array([0, 1, 2, 3, 127, 128, 511, 512, 1000, 1023, 1024, 1025, 1500, 2040, 2041, 2042, 2043, 2044,
                     2045, 2046, 2047, 77, 900, 1789])
    xs = I.widen(x[:, :, cols])
    y_ref, _ = oracle.short_conv(xs, w[cols], silu=True)
    check_y(host(y[:, :, cols]), y_ref, "bf16")
    dx_ref, dw_ref, _ = oracle.short_conv_bwd(xs, w[cols], dy[:, :, cols], silu=True)
    assert rel_max(host(r["dx"][:, :, cols]), dx_ref) < 2e-6
    assert rel_max(host(r["dw"][cols]), dw_ref) < 2e-5
