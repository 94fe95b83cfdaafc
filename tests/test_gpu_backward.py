"""Backward pass on the GPU (through the C-ABI) against the CPU fp64 oracle.

Tolerance for the bf16 backward.  The pages state none for gradients, so it
is derived from the arithmetic.
* Every gradient is a short chain of products whose operands are rounded to
  bf16 (relative error up to 2^-9 each) and accumulated in fp32.
* The result itself is rounded to bf16.
* About four such roundings give a relative L2 error of about 3.5e-3.
* dg is a reverse cumulative sum of terms that partly cancel.  That raises
  its relative error by the ratio of the summed magnitudes to the result,
  about 2 to 3.

Bound, per gradient tensor:
* rel-L2 <= 1e-2 (dg: 2e-2);
* max-abs <= 1e-2 * max|ref| (dg: 2e-2 * max|ref|).
"""

import numpy as np
import pytest
import torch

import oracle.kda_oracle as orc
from oracle.kda_backward import kda_backward
from gated_delta_rule_04_amd import inputs, kda
from tests._parity import errors, f64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
REL = {"dg": 2e-2}
MAXREL = {"dg": 2e-2}


def check_grad(tag, name, got, ref):
    got = f64(got)
    assert np.all(np.isfinite(got)), "%s %s: non-finite" % (tag, name)
    ma, rel = errors(got, ref)
    scale = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    print("PARITY %-34s %-6s max-abs %.3e (%.2e of max) rel-L2 %.3e" % (tag, name, ma, ma / scale, rel), flush=True)
    assert rel <= REL.get(name, 1e-2), "%s %s: rel-L2 %.3e" % (tag, name, rel)
    assert ma <= MAXREL.get(name, 1e-2) * scale, "%s %s: max-abs %.3e" % (tag, name, ma)


def run_gpu(d, ct):
    dev = lambda t: None if t is None else t.cuda()
    out = kda.chunk_bwd(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), dev(d["beta"]), dev(ct["do"]),
                        initial_state=dev(d.get("h0")), dht=dev(ct.get("dht")), cu_seqlens=dev(d.get("cu_seqlens")))
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


def run_oracle(d, ct):
    cu = d.get("cu_seqlens")
    return kda_backward(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(d["g"]), f64(d["beta"]), f64(ct["do"]),
                        h0=None if d.get("h0") is None else f64(d["h0"]),
                        dht=None if ct.get("dht") is None else f64(ct["dht"]),
                        cu_seqlens=None if cu is None else cu.numpy(), g_group=d["g_group"])


def case(B, T, H, dk, dv, gg=1, h0=True, dht=True, cu=None, seed=0, decay="config"):
    N = B if cu is None else len(cu) - 1
    d = inputs.make_prefill(B, T, H, dk, dv, "bf16", gg, seed=seed, h0=h0, cu_seqlens=cu, decay=decay)
    ct = inputs.make_cotangents(B, T, H, dk, dv, N, "bf16", seed=seed + 1000, final_state=dht, state_std=1.0)
    return d, ct


def compare(tag, d, ct):
    got = run_gpu(d, ct)
    ref = run_oracle(d, ct)
    for n in NAMES:
        check_grad(tag, n, got[n], ref[n])
    return got


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_head_sizes_ragged(dk, dv):
    # several chunks and a ragged tail, two sequences, h0 and dht
    d, ct = case(2, 201, 2, dk, dv, seed=dk + dv)
    compare("B2 T201 H2 dk%d dv%d" % (dk, dv), d, ct)


def test_single_chunk_no_states():
    d, ct = case(1, 64, 1, 64, 64, h0=False, dht=False, seed=1)
    compare("one chunk", d, ct)


@pytest.mark.parametrize("T", [1, 2, 63, 65, 127])
def test_short_and_boundary_lengths(T):
    # 32 heads, so that the whole-tensor criteria see a few dozen values even at T = 1
    d, ct = case(1, T, 32, 128, 128, seed=T)
    compare("T%d" % T, d, ct)


@pytest.mark.parametrize("dk", [64, 128])
def test_decay_groups_of_64(dk):
    d, ct = case(1, 256, 2, dk, 128, gg=64, seed=7 + dk)
    compare("g64 dk%d" % dk, d, ct)


def test_g64_matches_expanded_decay():
    """Compact g64 gives the group sums of the expanded run's dg, and the
    same other gradients (up to the bf16 rounding of the summed dg)."""
    d, ct = case(1, 190, 2, 128, 128, gg=64, seed=21)
    e = dict(d)
    e["g"] = d["g"].repeat_interleave(64, dim=-1).contiguous()
    e["g_group"] = 1
    a, b = run_gpu(d, ct), run_gpu(e, ct)
    for n in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert torch.equal(a[n], b[n]), n
    summed = f64(b["dg"]).reshape(1, 190, 2, 2, 64).sum(-1)
    ma, rel = errors(f64(a["dg"]), summed)
    assert rel <= 1e-2, rel


def test_packed_documents():
    cu = [0, 50, 50, 51, 180, 300]  # an empty document and a one-token one
    d, ct = case(1, 300, 2, 128, 128, cu=cu, seed=31)
    compare("varlen", d, ct)


def test_packed_documents_have_zero_cross_gradient():
    """Perturbing one document's inputs and cotangents leaves every gradient
    of the other documents bitwise unchanged."""
    cu = [0, 70, 70, 200, 333]
    d, ct = case(1, 333, 2, 128, 64, cu=cu, seed=41)
    a = run_gpu(d, ct)
    d2 = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ct2 = {k: v.clone() for k, v in ct.items()}
    sl = slice(70, 200)  # document 2
    for n in ("q", "k", "v", "beta", "g"):
        d2[n][:, sl] = d2[n][:, sl].flip(1)
    ct2["do"][:, sl] = -ct2["do"][:, sl]
    d2["h0"][2] = -d2["h0"][2]
    ct2["dht"][2] = 2 * ct2["dht"][2]
    b = run_gpu(d2, ct2)
    keep = torch.ones(333, dtype=torch.bool)
    keep[sl] = False
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(a[n][:, keep], b[n][:, keep]), n
        assert not torch.equal(a[n][:, sl], b[n][:, sl]), n
    for doc in (0, 1, 3):
        assert torch.equal(a["dh0"][doc], b["dh0"][doc])


def test_frozen_state_exact_zeros():
    """alpha = 1, beta = 0: the state never changes, so dk = dv = 0 exactly;
    dq, dbeta, dg, dh0 against the oracle (whose closed forms are pinned)."""
    d, ct = case(1, 150, 2, 128, 128, seed=51, decay="none")
    d["beta"].zero_()
    got = run_gpu(d, ct)
    assert torch.count_nonzero(got["dk"]) == 0 and torch.count_nonzero(got["dv"]) == 0
    ref = run_oracle(d, ct)
    for n in ("dq", "dbeta", "dg", "dh0"):
        check_grad("frozen", n, got[n], ref[n])


@pytest.mark.parametrize("which", ["do_only", "dht_only"])
def test_each_cotangent_path(which):
    """The output path and the final-state path separately: each one's
    gradients are checked alone, so a wrong term in either cannot hide
    behind the other."""
    d, ct = case(1, 230, 2, 128, 128, seed=61)
    if which == "do_only":
        ct["dht"] = None
    else:
        ct["do"].zero_()
    compare(which, d, ct)


def test_empty_sequence_passes_dht_through():
    d, ct = case(2, 0, 3, 64, 64, seed=71)
    got = run_gpu(d, ct)
    assert torch.equal(got["dh0"], ct["dht"])


def test_deterministic():
    d, ct = case(1, 300, 3, 128, 128, seed=81)
    a, b = run_gpu(d, ct), run_gpu(d, ct)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_caller_streams():
    """Results on two caller-made streams, with calls in flight on both at
    once, are bitwise those on torch's default stream."""
    d, ct = case(2, 333, 3, 128, 128, seed=83)
    ref = run_gpu(d, ct)
    g = {k: (None if t is None else t.cuda()) for k, t in
         (("q", d["q"]), ("k", d["k"]), ("v", d["v"]), ("g", d["g"]), ("beta", d["beta"]), ("h0", d.get("h0")),
          ("do", ct["do"]), ("dht", ct.get("dht")))}
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append(kda.chunk_bwd(g["q"], g["k"], g["v"], g["g"], g["beta"], g["do"], initial_state=g["h0"],
                                      dht=g["dht"]))
    torch.cuda.synchronize()
    for out in outs:
        for n in NAMES:
            assert torch.equal(out[n].cpu(), ref[n]), n


def test_forward_unchanged_by_state_keeping():
    """The backward's internal forward writes chunk states only: a forward
    call after it still matches the oracle (and the forward output path is
    independent of that option)."""
    d, ct = case(1, 200, 2, 128, 128, seed=91)
    run_gpu(d, ct)
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else v) for n, v in d.items()}
    o, ht = kda.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["h0"],
                          output_final_state=True)
    o_ref, h_ref = orc.kda_forward(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(d["g"]), f64(d["beta"]),
                                   h0=f64(d["h0"]))
    assert errors(o.cpu(), o_ref)[1] <= 5e-3 and errors(ht.cpu(), h_ref)[1] <= 5e-3


@pytest.mark.parametrize("decay", ["slow", "none"])
def test_long_reverse_chain(decay):
    """T = 4096 (64 chunks) with slow (alpha ~ 0.998) or no decay and small
    writes (beta / 10): the state cotangent then crosses every chunk of the
    reverse state pass almost undamped, so a wrong F^T or b stage anywhere in
    the chain shows in the early tokens' gradients and in dh0.  Every token
    of two heads, and dh0, against the oracle."""
    d, ct = case(1, 4096, 2, 128, 128, seed=4096 + len(decay), decay=decay)
    d["beta"] = (d["beta"].float() * 0.1).to(torch.bfloat16)
    compare("T4096 decay=%s beta/10" % decay, d, ct)


@pytest.mark.parametrize("chunk_sum", [-100.0, -300.0, -440.0])
@pytest.mark.parametrize("dk,dv,gg", [(128, 128, 1), (64, 64, 1), (128, 64, 64)])
def test_strong_decay(chunk_sum, dk, dv, gg):
    """Every third key channel (or decay group) decays by about e^chunk_sum
    over 64 tokens: far beyond what a chunk-start reference can carry in
    fp32 (e^{+-G} would reach e^{300}).  Two sequences with h0, dht and a
    ragged tail; every gradient against the oracle."""
    d, ct = case(2, 300, 2, dk, dv, gg=gg, seed=int(-chunk_sum) + dk + gg, decay="strong:%g" % chunk_sum)
    compare("strong %g dk%d dv%d gg%d" % (chunk_sum, dk, dv, gg), d, ct)


def test_strong_decay_packed_documents():
    cu = [0, 17, 17, 150, 333]
    d, ct = case(1, 333, 3, 128, 128, cu=cu, seed=303, decay="strong:-300")
    compare("strong -300 varlen", d, ct)


def test_mamba_style_gate_decay():
    """g from the gate -exp(A_log) softplus(f + dt_bias) with A_log = ln 16 (a
    Mamba-style A of 16): per-token log-decays near -3, single tokens near
    -50 and 64-token sums near -190.  The gate is evaluated by the prologue
    oracle in fp64 and rounded to bf16; the backward takes it as g."""
    import oracle.prologue as pro
    from tests._chunked_model import chunked_backward_blockref
    p = inputs.make_prologue(2, 400, 2, 128, 128, "bf16", seed=1616, h0=True, a_log_mean=float(np.log(16.0)))
    d, ct = case(2, 400, 2, 128, 128, seed=1617)
    g = pro.gate(f64(p["f"]), f64(p["A_log"]), f64(p["dt_bias"]))
    d["g"] = torch.from_numpy(g).float().to(torch.bfloat16)
    assert float(d["g"].float().sum(1).min()) < -800.0  # sums over 400 tokens
    got = run_gpu(d, ct)
    ref = run_oracle(d, ct)
    # dg here is a sum of terms that cancel to about a tenth of their size
    # (a token's decay reaches only a few tokens), so its relative error is
    # larger than elsewhere.  Its bound is derived from a float64 model of the
    # same block algebra with bf16 rounding at the GPU path's storage points:
    # twice that model's relative L2 error on these inputs.
    bf = lambda x: torch.from_numpy(np.asarray(x)).float().bfloat16().double().numpy()
    model = np.zeros(ref["dg"].shape)
    for b in range(2):
        for h in range(2):
            sel = lambda t: f64(t)[b, :, h]
            model[b, :, h] = chunked_backward_blockref(*(sel(d[n]) for n in ("q", "k", "v", "g", "beta")),
                                                       f64(d["h0"])[b, h], sel(ct["do"]), f64(ct["dht"])[b, h],
                                                       rnd=bf)["dg"]
    model_rel = errors(model, ref["dg"])[1]
    print("dg of the bf16 rounding model: rel-L2 %.3e" % model_rel)
    bound = max(2e-2, 2.0 * model_rel)
    for n in NAMES:
        if n == "dg":
            ma, rel = errors(f64(got[n]), ref[n])
            assert np.all(np.isfinite(f64(got[n])))
            print("PARITY %-34s %-6s max-abs %.3e rel-L2 %.3e (bound %.3e)" % ("A_log ln16 gate", n, ma, rel, bound),
                  flush=True)
            assert rel <= bound and ma <= 2e-2 * float(np.max(np.abs(ref[n])))
        else:
            check_grad("A_log ln16 gate", n, got[n], ref[n])


def test_kimi_k3_heads_full_chain():
    """At the bench's prefill shape (B=1, T=32768, H=96, dk=dv=128): every
    gradient of two heads over all 32,768 tokens, and their dh0, against the
    oracle run over the whole sequence (so the first tokens' gradients
    depend on the reverse pass through all 512 chunks); plus finiteness of
    every gradient of every head."""
    B, T, H, dk, dv = 1, 32768, 96, 128, 128
    d, ct = case(B, T, H, dk, dv, seed=2024, h0=False)
    got = run_gpu(d, ct)
    for n in NAMES:
        assert torch.isfinite(got[n]).all(), n
    heads = [5, 77]
    sel = lambda t: f64(t[:, :, heads])
    ref = kda_backward(*(sel(d[n]) for n in ("q", "k", "v", "g", "beta")), sel(ct["do"]),
                       dht=f64(ct["dht"][:, heads]))
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        check_grad("K3 heads all tokens", n, got[n][:, :, heads], ref[n])
        first = slice(0, 512)
        check_grad("K3 heads first 512", n, got[n][:, first][:, :, heads], ref[n][:, first])
    check_grad("K3 heads", "dh0", got["dh0"][:, heads], ref["dh0"])


def test_packed_documents_workload_full_size():
    """The packed-document workload at full size (65,536 tokens, 12 heads,
    about 46 documents of 16..8192 tokens), with seeded cotangents and no
    states.  Gradients never cross documents, so the oracle runs on whole
    documents alone: the three shortest and the longest, on two heads."""
    d = inputs.workload_prefill("varlen_bf16")
    cu = d["cu_seqlens"].numpy()
    N = len(cu) - 1
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    ct = inputs.make_cotangents(B, T, H, dk, dv, N, "bf16", seed=3003, final_state=True, state_std=1.0)
    got = run_gpu(d, ct)
    for n in NAMES:
        assert torch.isfinite(got[n]).all(), n
    lens = np.diff(cu)
    docs = list(np.argsort(lens, kind="stable")[:3]) + [int(np.argmax(lens))]
    heads = [3, 10]
    for doc in docs:
        a, b = int(cu[doc]), int(cu[doc + 1])
        sel = lambda t: f64(t[:, a:b][:, :, heads])
        ref = kda_backward(sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(d["g"]), sel(d["beta"]), sel(ct["do"]),
                           dht=f64(ct["dht"][doc:doc + 1, heads]))
        tag = "varlen doc %d (%d tokens)" % (doc, b - a)
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            check_grad(tag, n, got[n][:, a:b][:, :, heads], ref[n])
        check_grad(tag, "dh0", got["dh0"][doc:doc + 1, heads], ref["dh0"])


def test_decay_g64_workload_full_size():
    """The decay-g64 workload at full size (B=5, T=8192, H=12, dk=dv=128,
    one log-decay per 64 channels): every token of two sequences on two
    heads, and their dh0, against the oracle."""
    d = inputs.workload_prefill("mini1h_g64_bf16")
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    ct = inputs.make_cotangents(B, T, H, dk, dv, B, "bf16", seed=3004, final_state=True, state_std=1.0)
    got = run_gpu(d, ct)
    for n in NAMES:
        assert torch.isfinite(got[n]).all(), n
    heads = [0, 11]
    for b in (1, 4):
        sel = lambda t: f64(t[b:b + 1, :, heads])
        ref = kda_backward(*(sel(d[n]) for n in ("q", "k", "v", "g", "beta")), sel(ct["do"]),
                           dht=f64(ct["dht"][b:b + 1, heads]), g_group=64)
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            check_grad("g64 seq %d all tokens" % b, n, got[n][b:b + 1][:, :, heads], ref[n])
        check_grad("g64 seq %d" % b, "dh0", got["dh0"][b:b + 1, heads], ref["dh0"])


@pytest.mark.parametrize("packed,gg,dk", [(False, 1, 128), (True, 1, 128), (False, 64, 128), (True, 1, 64)])
def test_saved_states_pair_is_bitwise_the_plain_paths(packed, gg, dk):
    """kda_chunk_fwd_save returns the forward's o and ht bitwise, and
    kda_chunk_bwd_saved on its workspace the gradients of kda_chunk_bwd
    bitwise."""
    cu = [0, 70, 70, 200, 333] if packed else None
    d, ct = case(1 if packed else 2, 333 if packed else 201, 3, dk, 128, gg=gg, cu=cu, seed=97 + gg + dk)
    dev = lambda t: None if t is None else t.cuda()
    q, k, v, g, beta = (dev(d[n]) for n in ("q", "k", "v", "g", "beta"))
    h0, cs = dev(d["h0"]), dev(d["cu_seqlens"])
    o1, h1 = kda.chunk_fwd(q, k, v, g, beta, initial_state=h0, output_final_state=True, cu_seqlens=cs)
    o2, h2, ws = kda.chunk_fwd_save(q, k, v, g, beta, initial_state=h0, output_final_state=True, cu_seqlens=cs)
    a = kda.chunk_bwd(q, k, v, g, beta, dev(ct["do"]), initial_state=h0, dht=dev(ct["dht"]), cu_seqlens=cs)
    b = kda.chunk_bwd(q, k, v, g, beta, dev(ct["do"]), initial_state=h0, dht=dev(ct["dht"]), cu_seqlens=cs,
                      workspace=ws, states_saved=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n
