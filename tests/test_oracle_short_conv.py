"""Pins of the oracle's short convolution (the optional width-4 part of the
pre-mixer prep; "complex-kda-1.3B-100B" model card, Architecture: a short
convolution of width 4).  Each pin comes from outside the oracle's own loops:
an impulse response, numpy's convolve / correlate, document independence and
split composition, mathematical identities of SiLU, and central finite
differences of the reverse mode."""
import numpy as np
import pytest

import oracle

W = oracle.CONV_WIDTH


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_identity_filter_and_impulse_response():
    x = _rand(1, 2, 9, 5)
    w = np.zeros((5, W))
    w[:, 3] = 1.0                                 # the current token only
    y, _ = oracle.short_conv(x, w)
    assert np.array_equal(y, x)
    # an impulse at token 3 of channel 2 is answered by the taps in reverse
    # order on tokens 3..6 and by nothing before it (causal)
    w = _rand(2, 5, W)
    x = np.zeros((1, 10, 5))
    x[0, 3, 2] = 1.0
    y, _ = oracle.short_conv(x, w)
    assert np.all(y[0, :3] == 0) and np.all(y[0, 7:] == 0)
    for m in range(W):
        assert y[0, 3 + m, 2] == w[2, W - 1 - m]
    assert np.all(np.delete(y[0], 2, axis=1) == 0)


def test_matches_numpy_convolve_per_channel():
    x = _rand(3, 2, 40, 6)
    w = _rand(4, 6, W)
    y, st = oracle.short_conv(x, w)
    for b in range(2):
        for c in range(6):
            ref = np.convolve(x[b, :, c], w[c, ::-1])[:40]
            np.testing.assert_allclose(y[b, :, c], ref, rtol=1e-13, atol=1e-13)
        assert np.array_equal(st[b], x[b, -3:])


def test_silu_identities():
    # y = z sigmoid(z): silu(z) - silu(-z) = z, silu(0) = 0, and silu tends
    # to z (to 0) for large positive (negative) z
    z = np.linspace(-30, 30, 121)
    x = np.zeros((1, 121, 1))
    x[0, :, 0] = z
    w = np.array([[0.0, 0.0, 0.0, 1.0]])
    yp, _ = oracle.short_conv(x, w, silu=True)
    yn, _ = oracle.short_conv(-x, w, silu=True)
    np.testing.assert_allclose(yp[0, :, 0] - yn[0, :, 0], z, rtol=0, atol=1e-12)
    assert yp[0, 60, 0] == 0.0
    assert abs(yp[0, -1, 0] - 30.0) < 1e-11 and abs(yp[0, 0, 0]) < 1e-11


def test_documents_are_independent_and_windows_compose():
    x = _rand(5, 50, 4)
    w = _rand(6, 4, W)
    cu = np.array([0, 7, 7, 9, 50])
    s0 = _rand(7, 4, W - 1, 4)
    y, st = oracle.short_conv(x, w, cu_seqlens=cu, state0=s0, silu=True)
    for d in range(4):
        a, b = cu[d], cu[d + 1]
        yd, sd = oracle.short_conv(x[None, a:b], w, state0=s0[d:d + 1], silu=True)
        assert np.array_equal(y[a:b], yd[0])
        assert np.array_equal(st[d], sd[0])
    # the empty document hands its window straight on; a 2-token one keeps
    # one input of its history
    assert np.array_equal(st[1], s0[1])
    assert np.array_equal(st[2], np.concatenate([s0[2][2:], x[7:9]]))
    # zero history equals no history
    z0, _ = oracle.short_conv(x, w, cu_seqlens=cu, state0=np.zeros((4, W - 1, 4)))
    z1, _ = oracle.short_conv(x, w, cu_seqlens=cu)
    assert np.array_equal(z0, z1)
    # a sequence run in two parts, the window carried, equals one run
    xs = _rand(8, 1, 30, 3)
    ws = _rand(9, 3, W)
    y_all, st_all = oracle.short_conv(xs, ws, silu=True)
    y1, st1 = oracle.short_conv(xs[:, :11], ws, silu=True)
    y2, st2 = oracle.short_conv(xs[:, 11:], ws, state0=st1, silu=True)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y_all, rtol=0, atol=1e-14)
    assert np.array_equal(st2, st_all)


def test_decode_steps_equal_the_sequence():
    x = _rand(10, 3, 12, 5)
    w = _rand(11, 5, W)
    s0 = _rand(12, 3, W - 1, 5)
    y, st = oracle.short_conv(x, w, state0=s0, silu=True)
    win = s0
    for t in range(12):
        yt, win = oracle.short_conv_step(x[:, t], w, win, silu=True)
        np.testing.assert_allclose(yt, y[:, t], rtol=0, atol=1e-14)
    assert np.array_equal(win, st)


def test_linear_reverse_mode_is_a_correlation():
    x = _rand(13, 1, 25, 3)
    w = _rand(14, 3, W)
    dy = _rand(15, 1, 25, 3)
    s0 = _rand(16, 1, W - 1, 3)
    dx, dw, ds = oracle.short_conv_bwd(x, w, dy, state0=s0)
    for c in range(3):
        # dx_t = sum_m w[3 - m] dy_{t+m} (dy zero past the end)
        ref = np.correlate(np.concatenate([dy[0, :, c], np.zeros(W - 1)]), w[c, ::-1], "valid")
        full = np.concatenate([np.zeros(W - 1), dy[0, :, c]])
        np.testing.assert_allclose(dx[0, :, c], ref[:25], rtol=1e-13, atol=1e-13)
        # dw_j = sum_t dy_t x_{t-3+j} over the history-extended input
        xx = np.concatenate([s0[0, :, c], x[0, :, c]])
        np.testing.assert_allclose(dw[c], np.correlate(xx, dy[0, :, c], "valid"), rtol=1e-13, atol=1e-13)
        # the history's gradient: the taps that reach before the start
        np.testing.assert_allclose(ds[0, :, c], np.correlate(np.concatenate([full, np.zeros(W - 1)]),
                                                             w[c, ::-1], "valid")[:W - 1], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("silu", [False, True])
def test_reverse_mode_matches_finite_differences(silu):
    cu = np.array([0, 5, 6, 14])
    x = _rand(17, 14, 3)
    w = _rand(18, 3, W) * 0.7
    s0 = _rand(19, 3, W - 1, 3)
    dy = _rand(20, 14, 3)
    dx, dw, ds = oracle.short_conv_bwd(x, w, dy, cu_seqlens=cu, state0=s0, silu=silu)

    def L(x_, w_, s_):
        return float(np.sum(oracle.short_conv(x_, w_, cu_seqlens=cu, state0=s_, silu=silu)[0] * dy))

    h = 1e-6
    for arr, grad, name in ((x, dx, "x"), (w, dw, "w"), (s0, ds, "state0")):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            p, m = arr.copy(), arr.copy()
            p[i] += h
            m[i] -= h
            args_p = {"x": (p, w, s0), "w": (x, p, s0), "state0": (x, w, p)}[name]
            args_m = {"x": (m, w, s0), "w": (x, m, s0), "state0": (x, w, m)}[name]
            fd = (L(*args_p) - L(*args_m)) / (2 * h)
            assert abs(fd - grad[i]) < 1e-7 * max(1.0, abs(fd)), (name, i, fd, grad[i])
