"""kda_chunk_fwd_noalloc (the allocation-free prefill, its order table in the
library's static device array) against kda_chunk_fwd with a workspace, both
called through the C ABI on identical inputs: the outputs and final states
must be bitwise equal (the same kernels run), on two calls in a row, the
second with fewer documents and tokens than the first, so it runs on the
table the first call left behind.  The oracle is also checked on the second
call, to the bf16 tolerances."""

import ctypes

import numpy as np
import pytest
import torch

import oracle.kda_oracle as orc
from gated_delta_rule_04_amd import inputs, kda
from tests._parity import assert_close, f64, to_dev

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(d, o, ht):
    B, T, H, Dk = d["q"].shape
    Dv = d["v"].shape[-1]
    cu = d.get("cu_seqlens")
    N = B if cu is None else cu.numel() - 1
    dt = kda.KDA_BF16 if d["q"].dtype == torch.bfloat16 else kda.KDA_F32
    st = kda.lib().kda_chunk_fwd_noalloc(_p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["g"]), _p(d["beta"]),
                                         _p(d.get("h0")), _p(o), _p(ht), _p(cu), N, B, T, H, Dk, Dv, d["g_group"],
                                         dt, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, kda.lib().kda_status_str(st)


def _case(lens, H, seed):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return inputs.make_prefill(1, int(cu[-1]), H, 128, 128, seed=seed, h0=True, cu_seqlens=cu)


def test_noalloc_matches_workspace_call_twice():
    first = _case([700, 16, 1500, 64, 333, 2100], 4, seed=31)
    second = _case([130, 900, 47], 2, seed=32)
    for tag, d in (("first", first), ("second", second)):
        print("CASE noalloc %s tokens %d docs %d" % (tag, d["q"].shape[1], d["cu_seqlens"].numel() - 1), flush=True)
        dd = to_dev(d)
        o_ref, ht_ref = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], initial_state=dd["h0"],
                                      output_final_state=True, cu_seqlens=dd["cu_seqlens"])
        o = torch.full_like(o_ref, float("nan"))
        ht = torch.full_like(ht_ref, float("nan"))
        _noalloc(dd, o, ht)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), tag
        assert torch.equal(ht.view(torch.int32), ht_ref.view(torch.int32)), tag
    # the second (smaller) call against the oracle as well
    d = second
    ro, rh = orc.kda_forward(*(f64(d[n]) for n in ("q", "k", "v", "g", "beta")), h0=f64(d["h0"]),
                             cu_seqlens=d["cu_seqlens"].numpy())
    assert_close("noalloc second o", o.cpu(), ro, torch.bfloat16)
    assert_close("noalloc second ht", ht.cpu(), rh, torch.bfloat16)


def test_noalloc_dense_and_fp32():
    d = inputs.make_prefill(2, 300, 3, 64, 64, dtype="f32", seed=33, h0=True)
    dd = to_dev(d)
    o_ref, ht_ref = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], initial_state=dd["h0"],
                                  output_final_state=True)
    o = torch.empty_like(o_ref)
    ht = torch.empty_like(ht_ref)
    _noalloc(dd, o, ht)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
