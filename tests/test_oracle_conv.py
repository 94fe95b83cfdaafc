"""Pins of the short-convolution oracle (CPU only)."""

import sys

import numpy as np
import pytest

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


# ---------------------------------------------------------------- backward
from oracle.short_conv import short_conv_backward  # noqa: E402


def _conv_loss(x, w, c0, dy, dfin, cu=None):
    y, fin = short_conv_forward(x, w, conv0=c0, cu_seqlens=cu)
    return float(np.sum(dy * y) + np.sum(dfin * fin))


def test_backward_finite_differences_with_documents_and_states():
    # the loss is linear in x and c0 and bilinear in (x, w), so central
    # differences are exact up to rounding
    rng = np.random.default_rng(40)
    cu = np.array([0, 5, 5, 6, 19, 30])
    for W in (1, 2, 4):
        x = rng.standard_normal((1, 30, 3))
        w = rng.standard_normal((3, W))
        c0 = rng.standard_normal((5, W - 1, 3))
        dy = rng.standard_normal((1, 30, 3))
        dfin = rng.standard_normal((5, W - 1, 3))
        dx, dw, dc0 = short_conv_backward(x, w, dy, conv0=c0, dfinal=dfin, cu_seqlens=cu)
        for name, val, grad in (("x", x, dx), ("w", w, dw), ("c0", c0, dc0)):
            for _ in range(3):
                d = rng.standard_normal(val.shape)
                args = dict(x=x, w=w, c0=c0)
                args[name] = val + 1e-3 * d
                lp = _conv_loss(args["x"], args["w"], args["c0"], dy, dfin, cu)
                args[name] = val - 1e-3 * d
                lm = _conv_loss(args["x"], args["w"], args["c0"], dy, dfin, cu)
                assert abs((lp - lm) / 2e-3 - np.sum(grad * d)) <= 1e-9 * max(1.0, abs(lp)), (W, name)


def test_backward_is_the_adjoint_and_matches_numpy_correlate():
    # <dy, conv(x)> = <dx, x> with zero history; dx is the correlation of dy
    # with the reversed taps, cut to the sequence
    rng = np.random.default_rng(41)
    x = rng.standard_normal((2, 40, 3))
    w = rng.standard_normal((3, 4))
    dy = rng.standard_normal((2, 40, 3))
    dx, dw, _ = short_conv_backward(x, w, dy)
    y, _ = short_conv_forward(x, w)
    assert abs(np.sum(dy * y) - np.sum(dx * x)) <= 1e-10 * np.sum(np.abs(dy * y))
    for b in range(2):
        for c in range(3):
            ref = np.correlate(dy[b, :, c], w[c, ::-1], mode="full")[3:3 + 40]
            assert np.allclose(dx[b, :, c], ref, rtol=0, atol=1e-12)
    # dw[c, j] = sum_t dy[t] x[t - 3 + j] with zeros before the start
    for c in range(3):
        for j in range(4):
            s = 3 - j
            ref = sum(np.sum(dy[b, s:, c] * x[b, :40 - s, c]) for b in range(2))
            assert abs(dw[c, j] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_backward_width_one_and_documents_isolated():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((1, 12, 2))
    w = rng.standard_normal((2, 1))
    dy = rng.standard_normal((1, 12, 2))
    dx, dw, dc0 = short_conv_backward(x, w, dy)
    assert np.allclose(dx, dy * w[:, 0]) and np.allclose(dw[:, 0], np.sum(dy * x, axis=(0, 1)))
    assert dc0.shape == (1, 0, 2)
    # a cotangent in one document leaves every other document's dx at zero
    cu = np.array([0, 4, 9, 12])
    w = rng.standard_normal((2, 3))
    dy = np.zeros((1, 12, 2))
    dy[0, 5] = 1.0  # second token of document 1: reads its last history row and tokens 4, 5
    dx, _, dc0 = short_conv_backward(x, w, dy, conv0=rng.standard_normal((3, 2, 2)), cu_seqlens=cu)
    assert np.all(dx[0, :4] == 0) and np.all(dx[0, 6:] == 0) and np.all(dc0[[0, 2]] == 0)
    assert np.all(dx[0, 4:6] != 0) and np.all(dc0[1, 1] != 0) and np.all(dc0[1, 0] == 0)


def test_backward_mutants_fail_the_finite_difference_pin(monkeypatch):
    """Planted mistakes in the backward: each must fail the finite-difference pin."""
    import oracle.short_conv as sc
    real = sc.short_conv_backward

    def dfinal_ignored(x, w, dy, conv0=None, dfinal=None, cu_seqlens=None):
        return real(x, w, dy, conv0=conv0, dfinal=None, cu_seqlens=cu_seqlens)

    def history_dropped(x, w, dy, conv0=None, dfinal=None, cu_seqlens=None):
        dx, dw, dc0 = real(x, w, dy, conv0=conv0, dfinal=dfinal, cu_seqlens=cu_seqlens)
        return dx, dw, np.zeros_like(dc0)

    def taps_reversed(x, w, dy, conv0=None, dfinal=None, cu_seqlens=None):
        dx, dw, dc0 = real(x, w, dy, conv0=conv0, dfinal=dfinal, cu_seqlens=cu_seqlens)
        return dx, dw[:, ::-1], dc0

    for mutant in (dfinal_ignored, history_dropped, taps_reversed):
        monkeypatch.setattr(sys.modules[__name__], "short_conv_backward", mutant)
        with pytest.raises(AssertionError):
            test_backward_finite_differences_with_documents_and_states()
    monkeypatch.setattr(sys.modules[__name__], "short_conv_backward", real)
