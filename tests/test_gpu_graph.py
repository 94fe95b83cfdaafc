"""The entry points inside captured HIP graphs (torch.cuda.graph): the
library allocates nothing, syncs nothing and clears memory with kernels, so
a serving or training loop can capture its calls.  Each graph is replayed
several times with eager work in between, and every replay must equal the
eager calls bitwise (the kernels are deterministic)."""

import pytest
import torch

from gated_delta_rule_04_amd import inputs, kda

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    """fn() once on a side stream (warm-up, as torch's graph docs do), then captured."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_steps_in_a_graph():
    r = inputs.make_decode(4, 3, 128, 128, steps=8, seed=31)
    steps = [{n: t.cuda() for n, t in st.items()} for st in r["steps"]]
    S0 = r["state"].cuda()
    state_e = S0.clone()
    outs_e = []
    for st in steps:
        outs_e.append(kda.recurrent_step(st["q"], st["k"], st["v"], st["g"], st["beta"], state_e).clone())
    state = S0.clone()
    outs = [torch.empty_like(outs_e[0]) for _ in steps]

    def run():
        for st, o in zip(steps, outs):
            kda.recurrent_step(st["q"], st["k"], st["v"], st["g"], st["beta"], state, out=o)

    g = _capture(run)
    for rep in range(REPLAYS):
        state.copy_(S0)  # eager work between replays
        outs[0].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, state_e), rep
        for i in range(len(steps)):
            assert torch.equal(outs[i], outs_e[i]), (rep, i)


def test_packed_prefill_in_a_graph():
    cu = [0, 70, 70, 200, 333]
    d = inputs.make_prefill(1, 333, 3, 128, 128, "bf16", seed=32, h0=True, cu_seqlens=cu)
    dev = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in d.items()}
    args = [dev[n] for n in ("q", "k", "v", "g", "beta")]
    cs = dev["cu_seqlens"]
    o_e, h_e = kda.chunk_fwd(*args, initial_state=dev["h0"], output_final_state=True, cu_seqlens=cs)
    N = len(cu) - 1
    ws = torch.empty(kda.workspace_bytes(1, 333, 3, 128, 128, N, True, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(o_e)
    ht = torch.empty_like(h_e)

    def run():
        kda.chunk_fwd(*args, initial_state=dev["h0"], output_final_state=True, cu_seqlens=cs, out=o, final_state=ht,
                      workspace=ws)

    g = _capture(run)
    for rep in range(REPLAYS):
        o.fill_(1.0)
        ht.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(ht, h_e), rep


def test_training_pair_in_a_graph():
    d = inputs.make_prefill(2, 201, 3, 128, 128, "bf16", seed=33, h0=True)
    ct = inputs.make_cotangents(2, 201, 3, 128, 128, 2, "bf16", seed=34, state_std=1.0)
    dev = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in d.items()}
    args = [dev[n] for n in ("q", "k", "v", "g", "beta")]
    do, dht = ct["do"].cuda(), ct["dht"].cuda()
    o_e, h_e = kda.chunk_fwd(*args, initial_state=dev["h0"], output_final_state=True)
    gr_e = kda.chunk_bwd(*args, do, initial_state=dev["h0"], dht=dht)
    ws = torch.empty(kda.bwd_workspace_bytes(2, 201, 3, 128, 128, 2, False, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    o, ht = torch.empty_like(o_e), torch.empty_like(h_e)
    gr = {n: torch.empty_like(t) for n, t in gr_e.items()}

    def run():
        kda.chunk_fwd_save(*args, initial_state=dev["h0"], output_final_state=True, out=o, final_state=ht,
                           workspace=ws)
        kda.chunk_bwd(*args, do, initial_state=dev["h0"], dht=dht, workspace=ws, out=gr, states_saved=True)

    g = _capture(run)
    for rep in range(REPLAYS):
        for t in gr.values():
            t.zero_()
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(ht, h_e), rep
        for n, t in gr_e.items():
            assert torch.equal(gr[n], t), (rep, n)


def test_prologue_and_conv_backwards_in_a_graph():
    d = inputs.make_prologue(1, 150, 2, 128, 128, "bf16", seed=35, h0=True)
    ct = inputs.make_cotangents(1, 150, 2, 128, 128, 1, "bf16", seed=36, final_state=True, state_std=1.0)
    dev = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in d.items()}
    do, dht = ct["do"].cuda(), ct["dht"].cuda()
    pargs = [dev[n] for n in ("q_raw", "k_raw", "v", "f", "b_raw", "A_log", "dt_bias")]
    x = torch.randn((1, 300, 64), generator=torch.Generator().manual_seed(37)).bfloat16().cuda()
    w = (0.5 * torch.randn((64, 4), generator=torch.Generator().manual_seed(38))).bfloat16().cuda()
    dy = torch.randn((1, 300, 64), generator=torch.Generator().manual_seed(39)).bfloat16().cuda()
    pe = kda.chunk_bwd_prologue(*pargs, do, initial_state=dev["h0"], dht=dht)
    ce = kda.short_conv_bwd(x, w, dy)
    torch.cuda.synchronize()
    res = {}

    def run():
        res["p"] = kda.chunk_bwd_prologue(*pargs, do, initial_state=dev["h0"], dht=dht)
        res["c"] = kda.short_conv_bwd(x, w, dy)

    g = _capture(run)
    for rep in range(REPLAYS):
        for t in list(res["p"].values()) + list(res["c"].values()):
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in pe.items():
            assert torch.equal(res["p"][n], t), (rep, n)
        for n, t in ce.items():
            assert torch.equal(res["c"][n], t), (rep, n)
