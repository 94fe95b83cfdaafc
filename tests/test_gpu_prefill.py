"""Chunked prefill on the GPU (through the C-ABI) against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle.kda_oracle as orc
from gated_delta_rule_04_amd import inputs, kda
from tests._parity import assert_close, f64, to_dev

pytestmark = pytest.mark.gpu


def _oracle(d, heads=None, batches=None):
    """Oracle on the exact input values; optionally on a subset of heads/batch rows."""
    sel = lambda t: t
    q, k, v, g, beta = (f64(d[n]) for n in ("q", "k", "v", "g", "beta"))
    h0 = None if d.get("h0") is None else f64(d["h0"])
    if batches is not None:
        q, k, v, g, beta = (x[batches] for x in (q, k, v, g, beta))
        h0 = None if h0 is None else h0[batches]
    if heads is not None:
        q, k, v, g, beta = (x[:, :, heads] for x in (q, k, v, g, beta))
        h0 = None if h0 is None else h0[:, heads]
    cu = None if d.get("cu_seqlens") is None else d["cu_seqlens"].numpy()
    return orc.kda_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu, g_group=d["g_group"])


def _gpu(d, final=True):
    dd = to_dev(d)
    o, ht = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], initial_state=dd.get("h0"),
                          output_final_state=final, cu_seqlens=dd.get("cu_seqlens"))
    torch.cuda.synchronize()
    return o.cpu(), (ht.cpu() if ht is not None else None)


def _check(d, o, ht, heads=None, batches=None, tag=""):
    o_ref, h_ref = _oracle(d, heads=heads, batches=batches)
    og, hg = o, ht
    if batches is not None:
        og, hg = og[batches], hg[batches]
    if heads is not None:
        og, hg = og[:, :, heads], hg[:, heads]
    dt = d["q"].dtype
    assert_close(tag + " o", og, o_ref, dt)
    assert_close(tag + " ht", hg, h_ref, dt)


# ---------------------------------------------------------------- workloads
def test_tiny_f32():
    d = inputs.workload_prefill("tiny_f32")
    o, ht = _gpu(d)
    _check(d, o, ht, tag="tiny_f32")


def test_minikimi_bf16():
    d = inputs.workload_prefill("minikimi_bf16")
    o, ht = _gpu(d)
    _check(d, o, ht, tag="minikimi_bf16")


def test_mini1h_g64_bf16_full():
    # full-size launch; the oracle on every batch row and head over the whole length
    d = inputs.workload_prefill("mini1h_g64_bf16")
    o, ht = _gpu(d)
    _check(d, o, ht, tag="mini1h_g64 all rows and heads")


def test_varlen_bf16_full_and_packed_equals_separate():
    d = inputs.workload_prefill("varlen_bf16")
    o, ht = _gpu(d)
    _check(d, o, ht, tag="varlen all documents and heads")
    cu = d["cu_seqlens"].numpy()
    # separately launched documents give the same bits
    dd = to_dev(d)
    for n in (0, 1, len(cu) // 2, len(cu) - 2):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda t: t[:, a:b].contiguous()
        on, hn = kda.chunk_fwd(sl(dd["q"]), sl(dd["k"]), sl(dd["v"]), sl(dd["g"]), sl(dd["beta"]),
                               output_final_state=True)
        torch.cuda.synchronize()
        assert torch.equal(on.cpu(), o[:, a:b]), "document %d: packed != separate" % n
        assert torch.equal(hn.cpu()[0], ht[n]), "document %d final state: packed != separate" % n


# Heads of the K3 workload compared with the oracle: every residue mod 8 (the
# grid places unit u on XCD u % 8) and unit groups from both ends and the middle.
K3_HEADS = [0, 9, 18, 27, 36, 45, 54, 63, 95]


def test_k3_prefill_bf16_sampled():
    d = inputs.workload_prefill("k3_prefill_bf16")
    o, ht = _gpu(d)
    _check(d, o, ht, heads=K3_HEADS, tag="k3_prefill 9 heads")


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 33, 63, 64, 65, 100, 127, 128, 129, 191, 200])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_lengths(T, dtype):
    d = inputs.make_prefill(2, T, 3, 64, 64, dtype, 1, seed=100 + T, h0=True)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="T=%d %s" % (T, dtype))


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (128, 128), (64, 64)])
@pytest.mark.parametrize("g_group", [1, 64])
def test_head_dims_and_groups(dk, dv, g_group):
    d = inputs.make_prefill(2, 200, 2, dk, dv, "bf16", g_group, seed=7 + dk + dv + g_group, h0=True)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="dk=%d dv=%d gg=%d" % (dk, dv, g_group))


@pytest.mark.parametrize("dv", [64, 128])
def test_f32_dv(dv):
    d = inputs.make_prefill(1, 300, 2, 64, dv, "f32", 1, seed=41, h0=True)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="f32 dv=%d" % dv)


def test_g64_compact_equals_expanded():
    d = inputs.make_prefill(1, 257, 4, 128, 128, "bf16", 64, seed=3)
    o1, h1 = _gpu(d)
    e = dict(d)
    e["g"] = d["g"].repeat_interleave(64, dim=-1).contiguous()
    e["g_group"] = 1
    o2, h2 = _gpu(e)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("decay", ["slow", "none"])
def test_slow_and_no_decay_long(decay):
    d = inputs.make_prefill(1, 4096, 2, 128, 128, "bf16", 1, seed=9, decay=decay)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="decay=" + decay)


def test_split_equivalence():
    d = inputs.make_prefill(1, 700, 3, 128, 128, "bf16", 1, seed=12, h0=True)
    dd = to_dev(d)
    o, ht = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], initial_state=dd["h0"],
                          output_final_state=True)
    for t in (64, 300):
        sl = lambda x, a, b: x[:, a:b].contiguous()
        oa, ha = kda.chunk_fwd(*(sl(dd[n], 0, t) for n in ("q", "k", "v", "g", "beta")),
                               initial_state=dd["h0"], output_final_state=True)
        ob, hb = kda.chunk_fwd(*(sl(dd[n], t, 700) for n in ("q", "k", "v", "g", "beta")),
                               initial_state=ha, output_final_state=True)
        torch.cuda.synchronize()
        o_cat = torch.cat([oa, ob], dim=1)
        if t % 64 == 0:  # chunk-aligned split: identical arithmetic
            assert torch.equal(o_cat, o) and torch.equal(hb, ht)
        assert_close("split o", o_cat.cpu(), f64(o.cpu()), torch.bfloat16)


def test_final_state_may_alias_initial_state():
    d = inputs.make_prefill(2, 130, 2, 64, 64, "bf16", 1, seed=5, h0=True)
    dd = to_dev(d)
    h = dd["h0"].clone()
    o, ht = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], initial_state=h, final_state=h,
                          output_final_state=True)
    torch.cuda.synchronize()
    _check(d, o.cpu(), h.cpu(), tag="alias")


def test_deterministic():
    d = inputs.make_prefill(1, 1000, 4, 128, 128, "bf16", 1, seed=8)
    o1, h1 = _gpu(d)
    o2, h2 = _gpu(d)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_varlen_isolation_and_empty_documents():
    lens = [70, 0, 1, 130, 64, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = inputs.make_prefill(1, int(cu[-1]), 3, 128, 128, "bf16", 1, seed=21, h0=True, cu_seqlens=cu)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="varlen small")
    h0 = d["h0"]
    for n in (1, 5):
        assert torch.equal(ht[n], h0[n]), "empty document must return its initial state"
    # a NaN and a perturbation in document 3 leave every other document's bits unchanged
    j = 3
    a, b = int(cu[j]), int(cu[j + 1])
    d2 = dict(d)
    d2["v"] = d["v"].clone()
    d2["v"][:, a:b] += 1.0
    d2["q"] = d["q"].clone()
    d2["q"][:, a + 5] = float("nan")
    o2, ht2 = _gpu(d2)
    mask = torch.ones(o.shape[1], dtype=torch.bool)
    mask[a:b] = False
    assert torch.equal(o2[:, mask], o[:, mask])
    others = [n for n in range(len(lens)) if n != j]
    assert torch.equal(ht2[others], ht[others])


def test_empty_sequence_returns_initial_state():
    d = inputs.make_prefill(2, 0, 2, 64, 64, "bf16", 1, seed=1, h0=True)
    o, ht = _gpu(d)
    assert o.numel() == 0
    assert torch.equal(ht, d["h0"])


# ---------------------------------------------------------------- strong decay
@pytest.mark.parametrize("chunk_sum", [-100.0, -300.0, -440.0])
@pytest.mark.parametrize("dtype,dk,g_group", [("bf16", 128, 1), ("bf16", 64, 1), ("bf16", 128, 64),
                                              ("f32", 64, 1), ("f32", 128, 1)])
def test_strong_decay(chunk_sum, dtype, dk, g_group):
    """Every third key channel (or decay group) decays by about e^chunk_sum
    over 64 tokens (alpha ~ e^-1.6 or e^-4.7 per token), far beyond what one
    reference per 64-token chunk can hold in floats, inside the 16-token
    sub-block domain.  Against the oracle on every token and the final states,
    with initial states and a ragged tail."""
    d = inputs.make_prefill(2, 333, 3, dk, dk, dtype, g_group, seed=int(-chunk_sum) + dk + g_group, h0=True,
                            decay="strong:%g" % chunk_sum)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="strong %g %s dk%d gg%d" % (chunk_sum, dtype, dk, g_group))


def test_strong_decay_packed_documents():
    lens = [200, 1, 77, 0, 300]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = inputs.make_prefill(1, int(cu[-1]), 2, 128, 128, "bf16", 1, seed=77, h0=True, cu_seqlens=cu,
                            decay="strong:-300")
    o, ht = _gpu(d)
    _check(d, o, ht, tag="strong varlen")


# ---------------------------------------------------------------- fp32, 128 key channels
@pytest.mark.parametrize("T", [1, 15, 16, 17, 31, 32, 33, 100, 257])
def test_f32_dk128_ragged(T):
    d = inputs.make_prefill(2, T, 3, 128, 128, "f32", 1, seed=500 + T, h0=True)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="f32 dk128 T=%d" % T)


@pytest.mark.parametrize("dv,g_group", [(64, 1), (128, 64)])
def test_f32_dk128_shapes(dv, g_group):
    d = inputs.make_prefill(1, 600, 2, 128, dv, "f32", g_group, seed=600 + dv + g_group, h0=True)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="f32 dk128 dv%d gg%d" % (dv, g_group))


def test_f32_dk128_packed_documents():
    lens = [100, 0, 33, 64, 1, 250]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = inputs.make_prefill(1, int(cu[-1]), 2, 128, 128, "f32", 1, seed=601, h0=True, cu_seqlens=cu)
    o, ht = _gpu(d)
    _check(d, o, ht, tag="f32 dk128 varlen")
