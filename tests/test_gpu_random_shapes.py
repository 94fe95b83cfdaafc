"""Seeded random shapes against the oracle: prefill (bf16, and fp32 at
d_k = 64), the prefill with the fused prologue, decode steps and the backward, with random batch, length, head
count, head sizes, decay groups, initial states and packed documents
(including empty ones).  Each case prints its draw, so a failure names it.
Tolerances are the ones of the other parity tests."""

import numpy as np
import pytest
import torch

import oracle.kda_oracle as orc
import oracle.prologue as pro
from gated_delta_rule_04_amd import inputs, kda
from oracle.kda_backward import kda_backward
from tests._parity import assert_close, f64, to_dev
from tests.test_gpu_backward import NAMES, check_grad

pytestmark = pytest.mark.gpu


def _draw(seed, dks=(64, 128), max_t=260):
    rng = np.random.default_rng(seed)
    c = dict(dk=int(rng.choice(dks)), dv=int(rng.choice([64, 128])), gg=int(rng.choice([1, 64])),
             H=int(rng.integers(1, 4)), h0=bool(rng.integers(0, 2)))
    if c["gg"] > c["dk"]:
        c["gg"] = 1
    if rng.integers(0, 2):
        lens = [int(x) for x in rng.integers(0, 150, int(rng.integers(1, 6)))]
        if sum(lens) == 0:
            lens[-1] = 1
        c.update(B=1, cu=[0] + [int(x) for x in np.cumsum(lens)])
        c["T"] = c["cu"][-1]
    else:
        c.update(B=int(rng.integers(1, 4)), T=int(rng.integers(1, max_t)), cu=None)
    print("case seed %d: %s" % (seed, c), flush=True)
    return c


def _prefill(c, dtype, seed):
    return inputs.make_prefill(c["B"], c["T"], c["H"], c["dk"], c["dv"], dtype, c["gg"], seed=seed, h0=c["h0"],
                               cu_seqlens=c["cu"])


def _oracle_fwd(d):
    cu = None if d.get("cu_seqlens") is None else d["cu_seqlens"].numpy()
    return orc.kda_forward(*(f64(d[n]) for n in ("q", "k", "v", "g", "beta")),
                           h0=None if d.get("h0") is None else f64(d["h0"]), cu_seqlens=cu, g_group=d["g_group"])


def _gpu_fwd(d):
    dd = to_dev(d)
    o, ht = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], initial_state=dd.get("h0"),
                          output_final_state=True, cu_seqlens=dd.get("cu_seqlens"))
    torch.cuda.synchronize()
    return o.cpu(), ht.cpu()


@pytest.mark.parametrize("seed", range(16))
def test_random_prefill_bf16(seed):
    c = _draw(500 + seed)
    d = _prefill(c, "bf16", 500 + seed)
    o, ht = _gpu_fwd(d)
    o_ref, h_ref = _oracle_fwd(d)
    assert_close("random bf16 %d o" % seed, o, o_ref, torch.bfloat16)
    assert_close("random bf16 %d ht" % seed, ht, h_ref, torch.bfloat16)


@pytest.mark.parametrize("seed", range(6))
def test_random_prefill_f32(seed):
    c = _draw(600 + seed)
    d = _prefill(c, "f32", 600 + seed)
    o, ht = _gpu_fwd(d)
    o_ref, h_ref = _oracle_fwd(d)
    assert_close("random f32 %d o" % seed, o, o_ref, torch.float32)
    assert_close("random f32 %d ht" % seed, ht, h_ref, torch.float32)


@pytest.mark.parametrize("seed", range(8))
def test_random_prologue_forward(seed):
    """The fused gate/normalisation prologue in the prefill: random shapes,
    both input types, both head widths, decay groups and packed documents
    (rows past a document's end and partial chunks exercise the per-row
    gate mask and the norms of zero rows), against the prologue oracle."""
    rng = np.random.default_rng(900 + seed)
    dtype = "bf16" if seed % 2 == 0 else "f32"
    c = _draw(900 + seed)
    a_log = float(rng.choice([0.0, np.log(16.0)]))
    d = inputs.make_prologue(c["B"], c["T"], c["H"], c["dk"], c["dv"], dtype, g_group=c["gg"], seed=900 + seed,
                             h0=c["h0"], cu_seqlens=c["cu"], a_log_mean=a_log)
    print("prologue dtype %s A_log mean %.3f" % (dtype, a_log), flush=True)
    dd = to_dev(d)
    o, ht = kda.chunk_fwd_prologue(dd["q_raw"], dd["k_raw"], dd["v"], dd["f"], dd["b_raw"], dd["A_log"],
                                   dd["dt_bias"], initial_state=dd.get("h0"), output_final_state=True,
                                   cu_seqlens=dd.get("cu_seqlens"))
    torch.cuda.synchronize()
    cu = d.get("cu_seqlens")
    o_ref, h_ref = pro.kda_forward_prologue(
        f64(d["q_raw"]), f64(d["k_raw"]), f64(d["v"]), f64(d["f"]), f64(d["b_raw"]), f64(d["A_log"]),
        f64(d["dt_bias"]), h0=None if d.get("h0") is None else f64(d["h0"]),
        cu_seqlens=None if cu is None else cu.numpy(), g_group=d["g_group"])
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    assert_close("random prologue %d o" % seed, o.cpu(), o_ref, dt)
    assert_close("random prologue %d ht" % seed, ht.cpu(), h_ref, dt)


@pytest.mark.parametrize("seed", range(8))
def test_random_decode_steps(seed):
    rng = np.random.default_rng(700 + seed)
    N, H = int(rng.integers(1, 9)), int(rng.integers(1, 5))
    dk, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    gg = int(rng.choice([1, 64]))
    dtype = str(rng.choice(["bf16", "f32"]))
    print("case seed %d: N %d H %d dk %d dv %d gg %d %s" % (seed, N, H, dk, dv, gg, dtype), flush=True)
    r = inputs.make_decode(N, H, dk, dv, steps=3, dtype=dtype, g_group=gg, seed=700 + seed)
    state = r["state"].cuda()
    ref = f64(r["state"])
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    for i, st in enumerate(r["steps"]):
        o = kda.recurrent_step(*(st[n].cuda() for n in ("q", "k", "v", "g", "beta")), state)
        torch.cuda.synchronize()
        ref, o_ref = orc.kda_decode_step(ref, *(f64(st[n]) for n in ("q", "k", "v", "g", "beta")), g_group=gg)
        assert_close("random decode %d step %d o" % (seed, i), o.cpu(), o_ref, tdt)
        assert_close("random decode %d step %d S" % (seed, i), state.cpu(), ref, tdt)


@pytest.mark.parametrize("seed", range(8))
def test_random_backward(seed):
    c = _draw(800 + seed, max_t=200)
    d = _prefill(c, "bf16", 800 + seed)
    N = c["B"] if c["cu"] is None else len(c["cu"]) - 1
    ct = inputs.make_cotangents(c["B"], c["T"], c["H"], c["dk"], c["dv"], N, "bf16", seed=900 + seed,
                                final_state=bool(seed % 2 == 0), state_std=1.0)
    dev = lambda t: None if t is None else t.cuda()
    got = kda.chunk_bwd(*(dev(d[n]) for n in ("q", "k", "v", "g", "beta")), dev(ct["do"]),
                        initial_state=dev(d.get("h0")), dht=dev(ct.get("dht")), cu_seqlens=dev(d.get("cu_seqlens")))
    torch.cuda.synchronize()
    cu = d.get("cu_seqlens")
    ref = kda_backward(*(f64(d[n]) for n in ("q", "k", "v", "g", "beta")), f64(ct["do"]),
                       h0=None if d.get("h0") is None else f64(d["h0"]),
                       dht=None if ct.get("dht") is None else f64(ct["dht"]),
                       cu_seqlens=None if cu is None else cu.numpy(), g_group=d["g_group"])
    for n in NAMES:
        if n == "dh0" and d.get("h0") is None:
            continue
        check_grad("random bwd %d" % seed, n, got[n].cpu(), ref[n])


@pytest.mark.parametrize("seed", range(6))
def test_random_prologue_backward(seed):
    from tests.test_gpu_prologue_bwd import compare
    c = _draw(1200 + seed, max_t=180)
    d = inputs.make_prologue(c["B"], c["T"], c["H"], c["dk"], c["dv"], "bf16", g_group=c["gg"], seed=1200 + seed,
                             h0=True, cu_seqlens=c["cu"])
    N = c["B"] if c["cu"] is None else len(c["cu"]) - 1
    ct = inputs.make_cotangents(c["B"], c["T"], c["H"], c["dk"], c["dv"], N, "bf16", seed=1300 + seed,
                                final_state=True, state_std=1.0)
    compare("random prologue bwd %d" % seed, d, ct)


@pytest.mark.parametrize("seed", range(8))
def test_random_conv_backward(seed):
    from oracle.short_conv import short_conv_backward
    from tests.test_gpu_conv import _conv_bwd_check
    rng = np.random.default_rng(1400 + seed)
    W, C = int(rng.integers(1, 9)), 8 * int(rng.integers(1, 40))
    dt = torch.bfloat16 if rng.integers(0, 2) else torch.float32
    if rng.integers(0, 2):
        lens = [int(x) for x in rng.integers(0, 300, int(rng.integers(1, 7)))]
        if sum(lens) == 0:
            lens[-1] = 1
        cu = np.array([0] + list(np.cumsum(lens)), dtype=np.int32)
        B, T = 1, int(cu[-1])
    else:
        cu, B, T = None, int(rng.integers(1, 4)), int(rng.integers(1, 700))
    N = B if cu is None else len(cu) - 1
    states = bool(rng.integers(0, 2))
    print("case seed %d: W %d C %d %s B %d T %d docs %s states %s" % (seed, W, C, dt, B, T, None if cu is None
                                                                       else list(np.diff(cu)), states), flush=True)
    mk = lambda shape, s, scale=1.0: torch.from_numpy(
        (np.random.default_rng(s).standard_normal(shape) * scale).astype(np.float32)).to(dt)
    x, w, dy = mk((B, T, C), seed), mk((C, W), seed + 1, 0.5), mk((B, T, C), seed + 2)
    c0 = mk((N, W - 1, C), seed + 3) if states else None
    dfin = mk((N, W - 1, C), seed + 4) if states else None
    dev = lambda t: None if t is None else t.cuda()
    got = kda.short_conv_bwd(dev(x), dev(w), dev(dy), conv0=dev(c0), dconv_final=dev(dfin),
                             cu_seqlens=None if cu is None else torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    f = lambda t: None if t is None else t.float()
    ref = short_conv_backward(f(x), f(w), f(dy), conv0=f(c0), dfinal=f(dfin), cu_seqlens=cu)
    _conv_bwd_check("random conv bwd %d" % seed, got, ref, dt)
