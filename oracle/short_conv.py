"""CPU fp64 oracle of the short causal convolution (test infrastructure only:
used by tests/, never by the product path).

Sources: the miniKimiK3 card ("Limitations") -- order information reaches the
model only through KDA's decay and short convolutions plus the causal mask;
the Mini-K3-1H-mamba2 README (packed-document paragraph) -- convolution
history resets at every document boundary; the Mini-K3-1H cards list
convolution length as an ablation axis.

Readings (the pages give no formula): a depthwise causal convolution along
the token axis, per channel c with weights w[c, 0..W-1]:

    y[t, c] = sum_w w[c, w] * x[t - (W-1) + w, c]

with the W-1 positions before a sequence's first token taken from an initial
conv state (the inputs that preceded it) or zero; no bias, no activation.

Backward: the convolution is linear in x (and in the initial state) and in
the weights, so with L = <dy, y> + <dfinal, conv_final>:

    dx[t, c]      = sum_w w[c, w] dy[t + (W-1) - w, c]   (positions in the
                    same sequence) + dfinal where x[t] is one of the last W-1
    dw[c, w]      = sum_t dy[t, c] * ext[t + w, c]     (ext: history + x)
    dconv0[j, c]  = the same sums as dx for the W-1 history positions.
"""

import numpy as np


def _f64(a):
    return np.asarray(a.detach().cpu().double().numpy() if hasattr(a, "detach") else a, dtype=np.float64)


def _windowed(ext, w):
    """y[t] = sum_j w[:, j] * ext[t + j] for t = 0 .. len(ext) - W."""
    W = w.shape[1]
    L = ext.shape[0] - (W - 1)
    y = np.zeros((L, ext.shape[1]))
    for j in range(W):
        y += w[:, j][None, :] * ext[j:j + L]
    return y


def short_conv_forward(x, weight, conv0=None, cu_seqlens=None):
    """x: [B, T, C]; weight: [C, W]; conv0: [N, W-1, C] or None.
    Returns (y [B, T, C], conv_final [N, W-1, C]): conv_final holds each
    sequence's last W-1 inputs (earlier positions from conv0 or zeros)."""
    x = _f64(x)
    w = _f64(weight)
    B, T, C = x.shape
    W = w.shape[1]
    if cu_seqlens is not None:
        cu = [int(c) for c in np.asarray(cu_seqlens)]
        seqs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    else:
        seqs = [(b, 0, T) for b in range(B)]
    y = np.zeros((B, T, C))
    final = np.zeros((len(seqs), W - 1, C))
    for n, (b, s, e) in enumerate(seqs):
        hist = _f64(conv0)[n] if conv0 is not None else np.zeros((W - 1, C))
        ext = np.concatenate([hist, x[b, s:e]], axis=0)
        y[b, s:e] = _windowed(ext, w)
        final[n] = ext[ext.shape[0] - (W - 1):]
    return y, final


def short_conv_step(x, weight, conv_state):
    """One decode step: x [N, C]; weight [C, W]; conv_state [N, W-1, C].
    Returns (y [N, C], new_state [N, W-1, C])."""
    x = _f64(x)
    w = _f64(weight)
    st = _f64(conv_state)
    win = np.concatenate([st, x[:, None, :]], axis=1)  # [N, W, C]
    y = np.einsum("cw,nwc->nc", w, win)
    return y, win[:, 1:]


def short_conv_backward(x, weight, dy, conv0=None, dfinal=None, cu_seqlens=None):
    """Gradients of L = <dy, y> + <dfinal, conv_final> for short_conv_forward:
    returns (dx [B, T, C], dweight [C, W], dconv0 [N, W-1, C]).  dfinal
    [N, W-1, C] or None (zero)."""
    x = _f64(x)
    w = _f64(weight)
    dy = _f64(dy)
    B, T, C = x.shape
    W = w.shape[1]
    if cu_seqlens is not None:
        cu = [int(c) for c in np.asarray(cu_seqlens)]
        seqs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    else:
        seqs = [(b, 0, T) for b in range(B)]
    dx = np.zeros((B, T, C))
    dw = np.zeros((C, W))
    dc0 = np.zeros((len(seqs), W - 1, C))
    for n, (b, s, e) in enumerate(seqs):
        L = e - s
        hist = _f64(conv0)[n] if conv0 is not None else np.zeros((W - 1, C))
        ext = np.concatenate([hist, x[b, s:e]], axis=0)       # ext[i] feeds y[t] for i = t + j
        dext = np.zeros_like(ext)
        for j in range(W):
            dext[j:j + L] += w[:, j][None, :] * dy[b, s:e]
            dw[:, j] += np.sum(ext[j:j + L] * dy[b, s:e], axis=0)
        if dfinal is not None and W > 1:
            dext[ext.shape[0] - (W - 1):] += _f64(dfinal)[n]
        dx[b, s:e] = dext[W - 1:]
        dc0[n] = dext[:W - 1]
    return dx, dw, dc0
