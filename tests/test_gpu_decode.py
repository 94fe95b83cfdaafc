"""Recurrent decode step on the GPU (through the C-ABI) against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle.kda_oracle as orc
from gated_delta_rule_04_amd import inputs, kda
from tests._parity import assert_close, f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("g_group", [1, 64])
def test_decode_steps_full(dk, dv, dtype, g_group):
    r = inputs.make_decode(5, 3, dk, dv, steps=6, dtype=dtype, g_group=g_group, seed=dk + dv + g_group)
    state = r["state"].cuda()
    S = f64(r["state"])
    for s, st in enumerate(r["steps"]):
        dev = {n: st[n].cuda() for n in st}
        o = kda.recurrent_step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state)
        S, o_ref = orc.kda_decode_step(S, f64(st["q"]), f64(st["k"]), f64(st["v"]), f64(st["g"]),
                                       f64(st["beta"]), g_group=g_group)
        torch.cuda.synchronize()
        assert_close("o step %d" % s, o.cpu(), o_ref, st["q"].dtype)
    assert_close("state", state.cpu(), S, r["steps"][0]["q"].dtype)


def test_k3_decode_64_steps_sampled():
    """Full-size decode run (256 sequences x 96 heads x 128 x 128 fp32 state,
    64 steps, state carried); oracle on sampled (sequence, head) pairs."""
    r = inputs.workload_decode("k3_decode_bf16")
    state = r["state"].cuda()
    # sequences from both ends and the middle; heads on every residue mod 8
    # and from both ends of the head range
    seqs = np.array([0, 1, 127, 128, 254, 255])
    heads = np.array([0, 9, 18, 27, 36, 45, 54, 63, 95])
    S = f64(r["state"][seqs][:, heads])
    for s, st in enumerate(r["steps"]):
        dev = {n: st[n].cuda() for n in st}
        o = kda.recurrent_step(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state)
        sub = lambda t: f64(t[seqs][:, heads])
        S, o_ref = orc.kda_decode_step(S, sub(st["q"]), sub(st["k"]), sub(st["v"]), sub(st["g"]), sub(st["beta"]))
        if s % 16 == 0 or s == 63:
            torch.cuda.synchronize()
            assert_close("o step %d" % s, o.cpu()[seqs][:, heads], o_ref, torch.bfloat16)
    torch.cuda.synchronize()
    assert_close("final state", state.cpu()[seqs][:, heads], S, torch.bfloat16)


def test_decode_matches_prefill():
    """Stepping T tokens through the decode kernel agrees with one prefill."""
    d = inputs.make_prefill(2, 100, 2, 128, 128, "bf16", 1, seed=31, h0=True)
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else v) for n, v in d.items()}
    o, ht = kda.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["h0"],
                          output_final_state=True)
    state = dev["h0"].clone()
    outs = []
    for t in range(100):
        sl = lambda x: x[:, t].contiguous()
        outs.append(kda.recurrent_step(sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(dev["g"]), sl(dev["beta"]),
                                       state))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    assert_close("o decode vs prefill", o_dec.cpu(), f64(o.cpu()), torch.bfloat16)
    assert_close("state decode vs prefill", state.cpu(), f64(ht.cpu()), torch.bfloat16)


def test_decode_deterministic_and_strong_decay():
    """Bitwise repeatable; and any g (here g = -50: alpha ~ 0) is valid for decode."""
    r = inputs.make_decode(3, 2, 128, 128, steps=1, seed=2)
    st = {n: t.cuda() for n, t in r["steps"][0].items()}
    st["g"] = st["g"].clone()
    st["g"][0] = -50.0
    s1 = r["state"].cuda()
    s2 = r["state"].cuda()
    o1 = kda.recurrent_step(st["q"], st["k"], st["v"], st["g"], st["beta"], s1)
    o2 = kda.recurrent_step(st["q"], st["k"], st["v"], st["g"], st["beta"], s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    S, o_ref = orc.kda_decode_step(f64(r["state"]), *(f64(st[n].cpu()) for n in ("q", "k", "v", "g", "beta")))
    assert_close("o strong decay", o1.cpu(), o_ref, torch.bfloat16)
    assert_close("state strong decay", s1.cpu(), S, torch.bfloat16)
