"""Pins of the short-convolution oracle (CPU only)."""

import numpy as np

from oracle.short_conv import short_conv_forward, short_conv_step


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_matches_numpy_convolve_with_zero_history():
    # causal correlation = full convolution with the reversed kernel, cut to T
    x = _rand((2, 50, 3), 1)
    w = _rand((3, 4), 2)
    y, _ = short_conv_forward(x, w)
    for b in range(2):
        for c in range(3):
            ref = np.convolve(x[b, :, c], w[c, ::-1])[:50]
            assert np.allclose(y[b, :, c], ref, rtol=0, atol=1e-12)


def test_impulse_response_and_width_one():
    W, C, T = 5, 2, 20
    w = _rand((C, W), 3)
    x = np.zeros((1, T, C))
    x[0, 7, 1] = 1.0
    y, _ = short_conv_forward(x, w)
    for t in range(T):
        j = t - 7
        want = w[1, W - 1 - j] if 0 <= j < W else 0.0
        assert y[0, t, 1] == want and y[0, t, 0] == 0.0
    w1 = _rand((C, 1), 4)
    x = _rand((1, T, C), 5)
    y1, f1 = short_conv_forward(x, w1)
    assert np.array_equal(y1, x * w1[:, 0][None, None, :]) and f1.shape == (1, 0, C)


def test_documents_are_isolated_and_start_from_their_state():
    x = _rand((1, 30, 4), 6)
    w = _rand((4, 3), 7)
    cu = [0, 11, 11, 19, 30]  # an empty document in the middle
    c0 = _rand((4, 2, 4), 8)
    y, f = short_conv_forward(x, w, conv0=c0, cu_seqlens=cu)
    for n in range(4):
        s, e = cu[n], cu[n + 1]
        ys, fs = short_conv_forward(x[:, s:e], w, conv0=c0[n:n + 1])
        assert np.array_equal(y[:, s:e], ys) and np.array_equal(f[n], fs[0])
    assert np.array_equal(f[1], c0[1])  # an empty document keeps its initial state
    x2 = x.copy()
    x2[0, :11] += 5.0  # perturbing document 0 leaves the others unchanged
    y2, _ = short_conv_forward(x2, w, conv0=c0, cu_seqlens=cu)
    assert np.array_equal(y2[:, 11:], y[:, 11:])


def test_split_equivalence_and_decode_chain():
    x = _rand((2, 40, 5), 9)
    w = _rand((5, 4), 10)
    c0 = _rand((2, 3, 5), 11)
    y, f = short_conv_forward(x, w, conv0=c0)
    ya, fa = short_conv_forward(x[:, :17], w, conv0=c0)
    yb, fb = short_conv_forward(x[:, 17:], w, conv0=fa)
    assert np.allclose(np.concatenate([ya, yb], axis=1), y, atol=1e-14) and np.array_equal(fb, f)
    st = c0
    for t in range(40):
        yt, st = short_conv_step(x[:, t], w, st)
        assert np.allclose(yt, y[:, t], atol=1e-14)
    assert np.array_equal(st, f)
