"""Planted mistakes in the backward oracle (on the CPU): each plausible slip
in the reverse step must make the finite-difference pin fail.  This shows
the pin constrains every term of the reverse step."""

import numpy as np
import pytest

import oracle.kda_backward as bwd
import oracle.kda_oracle as orc

_real = bwd.reverse_step


def _mutant(kind):
    def step(Sp, q, k, v, g, beta, do, dS):
        a = np.exp(g)
        Sd = a[..., :, None] * Sp
        e = np.matmul(k[..., None, :], Sd)[..., 0, :]
        r = v - e
        u = beta[..., None] * r
        S_new = Sd + k[..., :, None] * u[..., None, :]
        read = Sd if kind == "dq_from_pre_write_state" else S_new
        dq = np.matmul(read, do[..., :, None])[..., 0]
        if kind != "no_output_cotangent_into_state":
            dS = dS + q[..., :, None] * do[..., None, :]
        du = np.matmul(k[..., None, :], dS)[..., 0, :]
        dk = np.matmul(dS, u[..., :, None])[..., 0]
        db = np.sum(du * (v if kind == "dbeta_without_erase" else r), axis=-1)
        dv = beta[..., None] * du if kind != "dv_without_beta" else du
        de = -beta[..., None] * du
        if kind == "wrong_sign_of_erase":
            de = -de
        if kind != "dk_without_erase_path":
            dk = dk + np.matmul(Sd, de[..., :, None])[..., 0]
        dSd = dS + k[..., :, None] * de[..., None, :] if kind != "state_without_erase_path" else dS
        dg = a * np.sum(dSd * Sp, axis=-1)
        if kind == "dg_without_alpha":
            dg = np.sum(dSd * Sp, axis=-1)
        if kind == "dg_from_decayed_state":
            dg = a * np.sum(dSd * Sd, axis=-1)
        dprev = a[..., :, None] * dSd if kind != "no_decay_on_state_cotangent" else dSd
        if kind == "decay_on_value_axis":
            dprev = dSd * np.swapaxes(a[..., :, None], -1, -2)[..., :, : dSd.shape[-1]] if a.shape[-1] >= dSd.shape[-1] else dSd
        return dq, dk, dv, dg, db, dprev
    return step


KINDS = ["dq_from_pre_write_state", "no_output_cotangent_into_state", "dbeta_without_erase", "dv_without_beta",
         "wrong_sign_of_erase", "dk_without_erase_path", "state_without_erase_path", "dg_without_alpha",
         "dg_from_decayed_state", "no_decay_on_state_cotangent", "decay_on_value_axis"]


def _fd_pin_holds():
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 5, 1, 4, 3
    z = rng.standard_normal((B, T, H, dk))
    q = z / np.linalg.norm(z, axis=-1, keepdims=True)
    z = rng.standard_normal((B, T, H, dk))
    k = z / np.linalg.norm(z, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.2, 0.9, (B, T, H))
    g = -rng.uniform(0.05, 0.6, (B, T, H, dk))
    h0 = rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dht = rng.standard_normal((B, H, dk, dv))
    gr = bwd.kda_backward(q, k, v, g, beta, do, h0=h0, dht=dht)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0")

    def loss(**kw):
        o, ht = orc.kda_forward(kw["q"], kw["k"], kw["v"], kw["g"], kw["beta"], h0=kw["h0"])
        return float(np.sum(do * o) + np.sum(dht * ht))

    eps = 1e-6
    for name, x in args.items():
        d = rng.standard_normal(x.shape)
        p, m = dict(args), dict(args)
        p[name], m[name] = x + eps * d, x - eps * d
        fd = (loss(**p) - loss(**m)) / (2 * eps)
        if abs(fd - float(np.sum(gr[names[name]] * d))) > 1e-7 * max(1.0, abs(fd)):
            return False
    return True


def test_real_reverse_step_passes():
    assert _fd_pin_holds()


@pytest.mark.parametrize("kind", KINDS)
def test_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(bwd, "reverse_step", _mutant(kind))
    assert not _fd_pin_holds(), kind
