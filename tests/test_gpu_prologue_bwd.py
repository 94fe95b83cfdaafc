"""Backward through the fused gate/normalisation prologue on the GPU (through
the C-ABI) against the CPU fp64 oracle (oracle.prologue.kda_backward_prologue).

Tolerances start from the backward's (derived in tests/test_gpu_backward.py
from the bf16 arithmetic): rel-L2 <= 1e-2 and max-abs <= 1e-2 * max|ref| per
gradient, 2e-2 for the decay-side gradients df, dA_log and d dt_bias, which
(like dg) are sums of terms that partly cancel.  Here the prepared q, k, g,
beta are stored in bf16 before the chunked backward runs on them, one more
rounding than the fused forward takes, and dA_log sums dg * g over every
token.  So each bound is the larger of that base value and twice the error
of a float64 model of the same steps with bf16 rounding at the GPU path's
storage points (the prepared inputs, then tests/_chunked_model.py's
block-referenced backward with its roundings), computed in the test on the
same inputs.  The parameter sums are also checked against the returned df
directly: d dt_bias is exactly the token sum of df."""

import numpy as np
import pytest
import torch

import oracle.prologue as pro
from gated_delta_rule_04_amd import inputs, kda
from tests._parity import errors, f64

pytestmark = pytest.mark.gpu

NAMES = ("dq_raw", "dk_raw", "dv", "df", "db_raw", "dA_log", "ddt_bias", "dh0")
LOOSE = {"df": 2e-2, "dA_log": 2e-2, "ddt_bias": 2e-2}


def _dev(t):
    return None if t is None else t.cuda()


def run(d, ct):
    out = kda.chunk_bwd_prologue(_dev(d["q_raw"]), _dev(d["k_raw"]), _dev(d["v"]), _dev(d["f"]), _dev(d["b_raw"]),
                                 _dev(d["A_log"]), _dev(d["dt_bias"]), _dev(ct["do"]),
                                 initial_state=_dev(d["h0"]), dht=_dev(ct["dht"]), cu_seqlens=_dev(d["cu_seqlens"]))
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


def oracle(d, ct):
    cu = d["cu_seqlens"]
    return pro.kda_backward_prologue(f64(d["q_raw"]), f64(d["k_raw"]), f64(d["v"]), f64(d["f"]), f64(d["b_raw"]),
                                     f64(d["A_log"]), f64(d["dt_bias"]), f64(ct["do"]),
                                     h0=None if d["h0"] is None else f64(d["h0"]),
                                     dht=None if ct["dht"] is None else f64(ct["dht"]),
                                     cu_seqlens=None if cu is None else cu.numpy(), g_group=d["g_group"])


def rounding_model(d, ct):
    """The prologue backward in float64 with bf16 rounding where the GPU path
    stores bf16: the prepared inputs, and the chunked backward's operands."""
    from tests._chunked_model import chunked_backward_blockref
    bf = lambda x: torch.from_numpy(np.asarray(x)).float().bfloat16().double().numpy()
    gg = d["g_group"]
    qr, kr, v, f, br = (f64(d[n]) for n in ("q_raw", "k_raw", "v", "f", "b_raw"))
    A, bias = f64(d["A_log"]), f64(d["dt_bias"])
    q, k, g, beta = (bf(x) for x in pro.prepare(qr, kr, f, br, A, bias))
    do, dht, h0 = f64(ct["do"]), f64(ct["dht"]), f64(d["h0"])
    B, T, H, dk = q.shape
    cu = None if d["cu_seqlens"] is None else [int(c) for c in d["cu_seqlens"].numpy()]
    seqs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)] if cu else [(b, 0, T) for b in range(B)]
    dq, dk_, dg = np.zeros(q.shape), np.zeros(k.shape), np.zeros(g.shape)
    dbeta, dv, dh0 = np.zeros(beta.shape), np.zeros(v.shape), np.zeros(h0.shape)
    for n, (b, s, e) in enumerate(seqs):
        for h in range(H):
            sl = lambda x: x[b, s:e, h]
            r = chunked_backward_blockref(sl(q), sl(k), sl(v), np.repeat(sl(g), gg, axis=-1), sl(beta), h0[n, h],
                                          sl(do), dht[n, h], rnd=bf)
            dq[b, s:e, h], dk_[b, s:e, h], dv[b, s:e, h], dbeta[b, s:e, h] = r["dq"], r["dk"], r["dv"], r["dbeta"]
            dg[b, s:e, h] = r["dg"].reshape(e - s, dk // gg, gg).sum(-1)
            dh0[n, h] = r["dh0"]
    out = pro.prologue_backward(qr, kr, f, br, A, bias, dq, dk_, dg, dbeta)
    out["dv"], out["dh0"] = dv, dh0
    return out


def compare(tag, d, ct):
    got, ref, model = run(d, ct), oracle(d, ct), rounding_model(d, ct)
    for n in NAMES:
        g = f64(got[n])
        assert np.all(np.isfinite(g)), "%s %s: non-finite" % (tag, n)
        ma, rel = errors(g, ref[n])
        mma, mrel = errors(model[n], ref[n])
        scale = max(1e-30, float(np.max(np.abs(ref[n]))))
        base = LOOSE.get(n, 1e-2)
        tol_rel, tol_max = max(base, 2.0 * mrel), max(base, 2.0 * mma / scale)
        print("PARITY %-30s %-8s max-abs %.3e (%.2e of max) rel-L2 %.3e  [model %.2e %.2e]"
              % (tag, n, ma, ma / scale, rel, mma / scale, mrel), flush=True)
        assert rel <= tol_rel and ma <= tol_max * scale, "%s %s: max-abs %.3e rel-L2 %.3e" % (tag, n, ma, rel)
    # d dt_bias is the token sum of df: per (head, group), within the bf16
    # rounding of the returned df (2^-8 of the summed magnitudes)
    dfs = f64(got["df"]).reshape(-1, *got["df"].shape[-2:])
    assert np.all(np.abs(f64(got["ddt_bias"]) - dfs.sum(0)) <= 2.0 ** -8 * np.abs(dfs).sum(0) + 1e-6)
    return got


def case(B, T, H, dk, dv, gg=1, cu=None, seed=0, a_log_mean=0.0):
    d = inputs.make_prologue(B, T, H, dk, dv, "bf16", g_group=gg, seed=seed, h0=True, cu_seqlens=cu,
                             a_log_mean=a_log_mean)
    N = B if cu is None else len(cu) - 1
    ct = inputs.make_cotangents(B, T, H, dk, dv, N, "bf16", seed=seed + 1000, final_state=True, state_std=1.0)
    return d, ct


@pytest.mark.parametrize("dk,dv,gg", [(64, 64, 1), (128, 128, 1), (128, 64, 64), (64, 128, 64)])
def test_prologue_bwd_head_sizes_and_groups(dk, dv, gg):
    d, ct = case(2, 150, 2, dk, dv, gg=gg, seed=dk + dv + gg)
    compare("prologue bwd dk%d dv%d gg%d" % (dk, dv, gg), d, ct)


def test_prologue_bwd_packed_documents_and_deterministic():
    cu = [0, 33, 33, 150, 301]
    d, ct = case(1, 301, 3, 128, 128, cu=cu, seed=77)
    got = compare("prologue bwd varlen", d, ct)
    again = run(d, ct)
    for n in NAMES:
        assert torch.equal(got[n], again[n]), n


def test_prologue_bwd_short_lengths():
    for T in (1, 17, 64, 65):
        d, ct = case(1, T, 4, 128, 128, seed=300 + T)
        compare("prologue bwd T%d" % T, d, ct)


def test_prologue_bwd_preallocated_out():
    """Gradients written into preallocated buffers (out=), twice in a row with
    the buffers holding the first call's values, equal the allocating call
    bitwise."""
    d, ct = case(2, 150, 2, 128, 128, seed=515)
    ref = run(d, ct)
    dev = {n: _dev(d[n]) for n in ("q_raw", "k_raw", "v", "f", "b_raw", "A_log", "dt_bias", "h0")}
    buf = {n: torch.full_like(ref[n], float("nan")).cuda() for n in NAMES}
    for _ in range(2):
        got = kda.chunk_bwd_prologue(dev["q_raw"], dev["k_raw"], dev["v"], dev["f"], dev["b_raw"], dev["A_log"],
                                     dev["dt_bias"], _dev(ct["do"]), initial_state=dev["h0"], dht=_dev(ct["dht"]),
                                     out=buf)
        torch.cuda.synchronize()
        for n in NAMES:
            assert got[n].data_ptr() == buf[n].data_ptr(), n
            assert torch.equal(got[n].cpu(), ref[n]), n
