"""Serving-pool decode step on the GPU (through the C-ABI) against the CPU
oracle: slot indirection, inactive sequences, bfloat16 and float16 state
pools, and the output gate."""

import numpy as np
import pytest
import torch

import oracle.kda_oracle as orc
from gated_delta_rule_04_amd import inputs, kda
from tests._parity import assert_close, f64

pytestmark = pytest.mark.gpu


def _dev(st):
    return {n: st[n].cuda() for n in st}


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
def test_pool_identity_slots_equal_plain_step(dk, dv):
    r = inputs.make_decode(6, 3, dk, dv, steps=1, dtype="bf16", g_group=1, seed=300 + dk)
    d = _dev(r["steps"][0])
    a = r["state"].cuda()
    b = r["state"].cuda()
    o1 = kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], a)
    o2 = kda.recurrent_step_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], b,
                                 torch.arange(6, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(a, b)


@pytest.mark.parametrize("dk,dv,g_group", [(64, 128, 1), (128, 64, 64), (128, 128, 1)])
def test_pool_permuted_and_inactive_slots(dk, dv, g_group):
    N, H, ns = 7, 2, 9
    r = inputs.make_decode(N, H, dk, dv, steps=1, dtype="bf16", g_group=g_group, seed=310 + dk + dv)
    st = r["steps"][0]
    d = _dev(st)
    pool0 = torch.from_numpy(np.random.default_rng(11).standard_normal((ns, H, dk, dv)) * 0.02).float()
    slots = np.array([5, -1, 0, 8, ns, 2, -7], dtype=np.int32)  # ns and negatives are inactive
    pool = pool0.cuda()
    o = kda.recurrent_step_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], pool,
                                torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    ref_pool, ref_o = orc.kda_decode_step_pool(f64(pool0), slots, f64(st["q"]), f64(st["k"]), f64(st["v"]),
                                               f64(st["g"]), f64(st["beta"]), g_group=g_group)
    active = [n for n in range(N) if 0 <= slots[n] < ns]
    assert_close("o active", o.cpu()[active], ref_o[active], torch.bfloat16)
    inactive = [n for n in range(N) if n not in active]
    assert torch.all(o.cpu()[inactive] == 0)
    used = sorted(int(slots[n]) for n in active)
    assert_close("pool used slots", pool.cpu()[used], ref_pool[used], torch.bfloat16)
    untouched = [s for s in range(ns) if s not in used]
    assert torch.equal(pool.cpu()[untouched], pool0[untouched])


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_pool_bf16_state_steps(dk, dv):
    N, H, steps = 5, 3, 12
    r = inputs.make_decode(N, H, dk, dv, steps=steps, dtype="bf16", g_group=1, seed=330 + dk + dv)
    ns = N + 2
    slots = np.array([3, 0, 6, 1, 4], dtype=np.int32)
    pool0 = torch.from_numpy(orc.round_bf16(np.random.default_rng(12).standard_normal((ns, H, dk, dv)) * 0.02))
    pool = pool0.to(torch.bfloat16).cuda()
    ref_pool = f64(pool0)
    sl = torch.from_numpy(slots).cuda()
    for s, st in enumerate(r["steps"]):
        d = _dev(st)
        o = kda.recurrent_step_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, sl)
        ref_pool, ref_o = orc.kda_decode_step_pool(ref_pool, slots, f64(st["q"]), f64(st["k"]), f64(st["v"]),
                                                   f64(st["g"]), f64(st["beta"]), state_bf16=True)
        torch.cuda.synchronize()
        assert_close("o step %d" % s, o.cpu(), ref_o, torch.bfloat16)
    assert_close("bf16 pool", pool.cpu()[slots], ref_pool[slots], torch.bfloat16)
    untouched = [s for s in range(ns) if s not in slots]
    assert torch.equal(pool.cpu()[untouched], pool0.to(torch.bfloat16)[untouched])


def test_k3_pool_bf16_state_sampled():
    """Full-size serving step: 256 sequences x 96 heads over a 300-slot bf16
    pool in shuffled slots, 4 steps; oracle on sampled (sequence, head) pairs."""
    r = inputs.workload_decode("k3_decode_bf16", steps=4)
    N, H = r["state"].shape[:2]
    ns = 300
    perm = np.random.default_rng(13).permutation(ns)[:N].astype(np.int32)
    pool_host = torch.zeros((ns, H) + tuple(r["state"].shape[2:]), dtype=torch.bfloat16)
    pool_host[torch.from_numpy(perm).long()] = r["state"].to(torch.bfloat16)
    pool = pool_host.cuda()
    sl = torch.from_numpy(perm).cuda()
    seqs, heads = np.array([0, 131, 255]), np.array([0, 47, 95])
    S = f64(pool_host[torch.from_numpy(perm[seqs]).long()][:, heads])
    for s, st in enumerate(r["steps"]):
        d = _dev(st)
        o = kda.recurrent_step_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, sl)
        sub = {n: f64(st[n][seqs][:, heads]) for n in st}
        S, o_ref = orc.kda_decode_step(S, sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"])
        S = orc.round_bf16(S)
        torch.cuda.synchronize()
        assert_close("k3 pool o step %d" % s, o.cpu()[seqs][:, heads], o_ref, torch.bfloat16)
    got = pool.cpu()[torch.from_numpy(perm[seqs]).long()][:, heads]
    assert_close("k3 pool state", got, S, torch.bfloat16)


@pytest.mark.parametrize("dk,dv,io", [(64, 64, "bf16"), (128, 128, "bf16"), (128, 64, "f32")])
def test_pool_f16_state_steps(dk, dv, io):
    N, H, steps = 5, 3, 12
    r = inputs.make_decode(N, H, dk, dv, steps=steps, dtype=io, g_group=1, seed=340 + dk + dv)
    ns = N + 2
    slots = np.array([6, 2, 0, 3, 5], dtype=np.int32)
    pool0 = torch.from_numpy(orc.round_f16(np.random.default_rng(14).standard_normal((ns, H, dk, dv)) * 0.02))
    pool = pool0.to(torch.float16).cuda()
    ref_pool = f64(pool0)
    sl = torch.from_numpy(slots).cuda()
    tol = torch.bfloat16 if io == "bf16" else torch.float16
    for s, st in enumerate(r["steps"]):
        d = _dev(st)
        o = kda.recurrent_step_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, sl)
        ref_pool, ref_o = orc.kda_decode_step_pool(ref_pool, slots, f64(st["q"]), f64(st["k"]), f64(st["v"]),
                                                   f64(st["g"]), f64(st["beta"]), state_dtype="f16")
        torch.cuda.synchronize()
        assert_close("o step %d" % s, o.cpu(), ref_o, torch.bfloat16)
    assert_close("f16 pool", pool.cpu()[slots], ref_pool[slots], tol)
    untouched = [s for s in range(ns) if s not in slots]
    assert torch.equal(pool.cpu()[untouched], pool0.to(torch.float16)[untouched])


@pytest.mark.parametrize("sdt,io", [(torch.float32, "bf16"), (torch.bfloat16, "bf16"), (torch.float32, "f32")])
def test_pool_output_gate(sdt, io):
    N, H, dk, dv, ns = 6, 2, 128, 128, 8
    r = inputs.make_decode(N, H, dk, dv, steps=1, dtype=io, g_group=1, seed=350)
    st = r["steps"][0]
    d = _dev(st)
    zt = torch.bfloat16 if io == "bf16" else torch.float32
    z = torch.from_numpy(np.random.default_rng(15).standard_normal((N, H, dv)) * 2).to(zt)
    slots = np.array([7, -1, 0, 3, ns, 5], dtype=np.int32)
    sl = torch.from_numpy(slots).cuda()
    base = torch.from_numpy(np.random.default_rng(16).standard_normal((ns, H, dk, dv)) * 0.02).to(sdt)
    pool_g, pool_n, pool_0 = base.cuda(), base.cuda(), base.cuda()
    o_g = kda.recurrent_step_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], pool_g, sl, o_gate=z.cuda())
    o_n = kda.recurrent_step_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], pool_n, sl)
    o_0 = kda.recurrent_step_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], pool_0, sl,
                                  o_gate=torch.zeros((N, H, dv), dtype=zt, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(pool_g, pool_n) and torch.equal(pool_0, pool_n)  # the gate never reaches the state
    assert torch.equal(o_0, o_n / 2)                                     # sigmoid(0) = 1/2, exact halving
    ref_pool, ref_o = orc.kda_decode_step_pool(f64(base), slots, f64(st["q"]), f64(st["k"]), f64(st["v"]),
                                               f64(st["g"]), f64(st["beta"]),
                                               state_dtype="bf16" if sdt == torch.bfloat16 else "f32",
                                               o_gate=f64(z))
    active = [n for n in range(N) if 0 <= slots[n] < ns]
    assert_close("gated o", o_g.cpu()[active], ref_o[active], torch.bfloat16 if io == "bf16" else torch.float32)
    assert torch.all(o_g.cpu()[[n for n in range(N) if n not in active]] == 0)


SDT_NAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("g_group", [1, 64])
@pytest.mark.parametrize("sdt", [torch.float32, torch.bfloat16, torch.float16])
def test_pool_prologue(sdt, g_group, io):
    """Raw projections into a pool: identity slots with an fp32 pool are
    bitwise the plain prologue step; permuted and inactive slots, every pool
    state type, both decay groupings (the gate index h * (Dk / g_group) +
    channel / g_group), both input types and the output gate against the
    oracle."""
    import oracle.prologue as pro
    N, H, dk, dv, ns = 5, 3, 128, 64, 7
    d = inputs.make_prologue(1, N, H, dk, dv, io, g_group=g_group, seed=60 + g_group)
    q, k, v, f, b = (d[n][0] for n in ("q_raw", "k_raw", "v", "f", "b_raw"))
    dev = lambda t: t.cuda()
    A, D = dev(d["A_log"]), dev(d["dt_bias"])
    iot = torch.bfloat16 if io == "bf16" else torch.float32
    base = torch.from_numpy(np.random.default_rng(17).standard_normal((ns, H, dk, dv)) * 0.02).to(sdt)
    print("CASE pool prologue state %s g_group %d io %s" % (SDT_NAME[sdt], g_group, io), flush=True)
    if sdt == torch.float32:
        a, p = base[:N].clone().cuda(), base[:N].clone().cuda()
        o1 = kda.recurrent_step_prologue(dev(q), dev(k), dev(v), dev(f), dev(b), A, D, a)
        o2 = kda.recurrent_step_pool_prologue(dev(q), dev(k), dev(v), dev(f), dev(b), A, D, p,
                                              torch.arange(N, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(a, p)
    slots = np.array([6, -1, 2, 0, 4], dtype=np.int32)
    z = torch.from_numpy(np.random.default_rng(18).standard_normal((N, H, dv))).to(iot)
    pool = base.cuda()
    o = kda.recurrent_step_pool_prologue(dev(q), dev(k), dev(v), dev(f), dev(b), A, D, pool,
                                         torch.from_numpy(slots).cuda(), o_gate=z.cuda())
    torch.cuda.synchronize()
    ref_pool, ref_o = pro.kda_decode_step_pool_prologue(
        f64(base), slots, f64(q), f64(k), f64(v), f64(f), f64(b), f64(d["A_log"]), f64(d["dt_bias"]),
        g_group=g_group, state_dtype=SDT_NAME[sdt], o_gate=f64(z))
    active = [n for n in range(N) if 0 <= slots[n] < ns]
    assert_close("pool prologue o", o.cpu()[active], ref_o[active], iot)
    assert torch.all(o.cpu()[1] == 0)
    used = sorted(int(slots[n]) for n in active)
    st_tol = torch.float32 if (sdt == torch.float32 and io == "f32") else torch.bfloat16
    assert_close("pool prologue state", pool.cpu()[used], ref_pool[used], st_tol)
    untouched = [s for s in range(ns) if s not in used]
    assert torch.equal(pool.cpu()[untouched], base[untouched])
