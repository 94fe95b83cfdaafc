"""The C-ABI library on the host: it loads, exports every declared symbol, and
rejects invalid arguments with its status codes before any HIP call (so these
run without a GPU and make no compute call)."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_04_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL, SHAPE, DTYPE, WORKSPACE, UNSUPPORTED = 0, 1, 2, 3, 4, 5

pytestmark = pytest.mark.skipif(not os.path.exists(kda.LIB_PATH), reason="libkda.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(kda.EXPORTED), names
    L = ctypes.CDLL(kda.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = kda.lib()
    assert L.kda_abi_version() == 10 == kda.ABI_VERSION
    for s in range(7):
        assert L.kda_status_str(s).decode().startswith(("KDA_OK", "KDA_ERR"))
    assert L.kda_status_str(99)


P = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def fwd(q=P, k=P, v=P, g=P, beta=P, h0=None, o=P, ht=None, cu=None, N=1, B=1, T=64, H=1, Dk=64, Dv=64, gg=1, dt=1,
        ws=None, wsb=0):
    return kda.lib().kda_chunk_fwd(q, k, v, g, beta, h0, o, ht, cu, N, B, T, H, Dk, Dv, gg, dt, ws, wsb, None)


def test_chunk_fwd_validation():
    assert fwd(dt=7) == DTYPE
    assert fwd(T=-1) == SHAPE
    assert fwd(H=0) == SHAPE
    assert fwd(Dk=96) == UNSUPPORTED
    assert fwd(Dv=256) == UNSUPPORTED
    assert fwd(gg=32) == UNSUPPORTED
    assert fwd(N=2, B=1) == SHAPE                     # without cu_seqlens N must equal B
    assert fwd(cu=P, B=2, N=2) == SHAPE               # varlen needs B == 1
    assert fwd(q=None) == NULL
    assert fwd(o=None) == NULL
    assert fwd(cu=P, N=3, ws=None, wsb=0) == WORKSPACE
    need = kda.lib().kda_chunk_fwd_workspace_bytes(1, 64, 1, 64, 64, 3, 1, 1)
    assert need >= 3 * 4
    assert fwd(cu=P, N=3, ws=P, wsb=need - 1) == WORKSPACE
    assert kda.lib().kda_chunk_fwd_workspace_bytes(1, 64, 1, 64, 64, 1, 0, 1) == 0
    assert fwd(B=2 ** 30, T=2 ** 30, N=2 ** 30) == SHAPE  # size overflow
    assert fwd(H=65536) == SHAPE                      # a chunk span must fit 32-bit byte offsets
    assert fwd(H=65535, B=0, T=0, N=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK


def fwd_noalloc(q=P, k=P, v=P, g=P, beta=P, h0=None, o=P, ht=None, cu=None, N=1, B=1, T=64, H=1, Dk=64, Dv=64,
                gg=1, dt=1):
    return kda.lib().kda_chunk_fwd_noalloc(q, k, v, g, beta, h0, o, ht, cu, N, B, T, H, Dk, Dv, gg, dt, None)


def test_chunk_fwd_noalloc_validation():
    # the checks of kda_chunk_fwd, minus the workspace, all before any HIP call
    assert fwd_noalloc(dt=7) == DTYPE
    assert fwd_noalloc(T=-1) == SHAPE
    assert fwd_noalloc(Dk=96) == UNSUPPORTED
    assert fwd_noalloc(cu=P, B=2, N=2) == SHAPE
    assert fwd_noalloc(cu=P, N=3, q=None) == NULL
    # the static order table holds KDA_NOALLOC_MAX_SEQS documents
    text = open(HEADER).read()
    limit = int(re.search(r"#define KDA_NOALLOC_MAX_SEQS (\d+)", text).group(1))
    assert limit == 65536
    assert fwd_noalloc(cu=P, N=limit + 1, T=limit + 1) == WORKSPACE
    assert fwd_noalloc(cu=P, N=2 ** 31 - 1) == WORKSPACE
    # nothing to launch: no device state is touched
    assert fwd_noalloc(cu=P, N=0, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK
    assert fwd_noalloc(N=0, B=0, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK


def test_chunk_fwd_nothing_to_do_is_ok_without_gpu():
    # no sequences: nothing is launched
    assert fwd(N=0, B=0, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK
    # tokens absent and no final state requested: nothing to launch
    assert fwd(N=2, B=2, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK


def test_recurrent_step_validation():
    L = kda.lib()
    step = lambda q=P, state=P, N=1, H=1, Dk=64, Dv=64, gg=1, dt=1: L.kda_recurrent_step(
        q, P, P, P, P, state, P, N, H, Dk, Dv, gg, dt, None)
    assert step(dt=2) == DTYPE
    assert step(N=-1) == SHAPE
    assert step(H=0) == SHAPE
    assert step(Dk=32) == UNSUPPORTED
    assert step(gg=2) == UNSUPPORTED
    assert step(q=None) == NULL
    assert step(state=None) == NULL
    assert step(N=0, q=None, state=None) == OK


def test_recurrent_step_pool_validation():
    L = kda.lib()
    step = lambda q=P, pool=P, slots=P, ns=4, N=1, H=1, Dk=64, Dv=64, gg=1, dt=1, sdt=1: L.kda_recurrent_step_pool(
        q, P, P, P, P, pool, slots, ns, P, None, N, H, Dk, Dv, gg, dt, sdt, None)
    assert step(dt=2) == DTYPE                        # float16 is a pool state type only
    assert step(sdt=5) == DTYPE
    assert step(sdt=2, N=0, q=None, pool=None, slots=None) == OK  # a float16 pool is accepted
    assert step(N=-1) == SHAPE
    assert step(H=0) == SHAPE
    assert step(ns=-1) == SHAPE
    assert step(Dv=96) == UNSUPPORTED
    assert step(gg=128) == UNSUPPORTED
    assert step(q=None) == NULL
    assert step(slots=None) == NULL
    assert step(pool=None) == NULL                    # a pool is required when num_slots > 0
    assert step(N=0, q=None, pool=None, slots=None) == OK


def test_recurrent_step_pool_prologue_validation():
    L = kda.lib()
    step = lambda q=P, A=P, pool=P, slots=P, ns=4, N=1, H=1, dt=1, sdt=1: L.kda_recurrent_step_pool_prologue(
        q, P, P, P, P, A, P, pool, slots, ns, P, None, N, H, 64, 64, 1, dt, sdt, None)
    assert step(dt=2) == DTYPE
    assert step(sdt=5) == DTYPE
    assert step(A=None) == NULL
    assert step(q=None) == NULL
    assert step(pool=None) == NULL
    assert step(H=0) == SHAPE
    assert step(N=0, q=None, A=None, pool=None, slots=None) == OK


def test_chunk_bwd_validation():
    L = kda.lib()

    def bwd(q=P, do=P, dq=P, dg=P, cu=None, N=1, B=1, T=64, H=1, Dk=64, Dv=64, gg=1, dt=1, ws=P, wsb=None):
        if wsb is None:
            wsb = L.kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, N, int(cu is not None), dt)
        return L.kda_chunk_bwd(q, P, P, P, P, None, do, None, dq, P, P, dg, P, None, cu, N, B, T, H, Dk, Dv, gg, dt,
                               ws, wsb, None)

    assert bwd(dt=7) == DTYPE
    assert bwd(T=-1) == SHAPE
    assert bwd(H=65536, wsb=0) == SHAPE
    assert bwd(Dk=96) == UNSUPPORTED
    assert bwd(dt=0) == UNSUPPORTED                   # the backward is bf16 only
    assert bwd(N=2, B=1) == SHAPE
    assert bwd(cu=P, B=2, N=2) == SHAPE
    assert bwd(do=None) == NULL
    assert bwd(dq=None) == NULL
    assert bwd(dg=None) == NULL
    need = L.kda_chunk_bwd_workspace_bytes(1, 64, 1, 64, 64, 1, 0, 1)
    # chunk states, F^T, b and the state cotangents for (64/64 + 1 + 1) slots
    assert need >= 3 * (64 * 64 * 2 * 4)
    assert bwd(wsb=need - 1) == WORKSPACE
    assert bwd(ws=None) == WORKSPACE
    assert bwd(ws=ctypes.c_void_p(0x1008)) == WORKSPACE  # not 256-byte aligned
    assert L.kda_chunk_bwd_workspace_bytes(1, -1, 1, 64, 64, 1, 0, 1) == 0


def test_prologue_validation():
    L = kda.lib()
    pf = lambda dt=1, A=P, Dk=64: L.kda_chunk_fwd_prologue(P, P, P, P, P, A, P, None, P, None, None, 1, 1, 64, 1, Dk,
                                                           64, 1, dt, None, 0, None)
    assert pf(dt=9) == DTYPE
    assert pf(A=None) == NULL
    assert pf(Dk=32) == UNSUPPORTED
    ps = lambda dt=1, A=P, N=1, H=1, q=P: L.kda_recurrent_step_prologue(q, P, P, P, P, A, P, P, P, N, H, 64, 64, 1,
                                                                        dt, None)
    assert ps(dt=9) == DTYPE
    assert ps(H=0) == SHAPE
    assert ps(A=None) == NULL
    assert ps(q=None) == NULL
    assert ps(N=0, q=None, A=None) == OK


def test_saved_pair_validation():
    L = kda.lib()
    need = L.kda_chunk_bwd_workspace_bytes(1, 64, 1, 64, 64, 1, 0, 1)
    fs = lambda o=P, dt=1, ws=P, wsb=need: L.kda_chunk_fwd_save(P, P, P, P, P, None, o, None, None, 1, 1, 64, 1, 64,
                                                                 64, 1, dt, ws, wsb, None)
    assert fs(dt=0) == UNSUPPORTED
    assert fs(o=None) == NULL
    assert fs(wsb=need - 1) == WORKSPACE
    assert fs(ws=None) == WORKSPACE
    bs = lambda do=P, dt=1, wsb=need: L.kda_chunk_bwd_saved(P, P, P, P, P, None, do, None, P, P, P, P, P, None, None,
                                                            1, 1, 64, 1, 64, 64, 1, dt, P, wsb, None)
    assert bs(dt=0) == UNSUPPORTED
    assert bs(do=None) == NULL
    assert bs(wsb=need - 1) == WORKSPACE


def test_chunk_bwd_prologue_validation():
    L = kda.lib()
    need = L.kda_chunk_bwd_prologue_workspace_bytes(1, 64, 1, 64, 64, 1, 0, 1, 1)
    assert need > L.kda_chunk_bwd_workspace_bytes(1, 64, 1, 64, 64, 1, 0, 1)
    assert L.kda_chunk_bwd_prologue_workspace_bytes(1, 64, 1, 96, 64, 1, 0, 1, 1) == 0

    def pb(qr=P, A=P, dA=P, dt=1, gg=1, ws=P, wsb=need, Dk=64, N=1, B=1, T=64, H=1, cu=None):
        return L.kda_chunk_bwd_prologue(qr, P, P, P, P, A, P, None, P, None, P, P, P, P, P, dA, P, None, cu, N, B, T,
                                        H, Dk, 64, gg, dt, ws, wsb, None)

    assert pb(dt=7) == DTYPE
    assert pb(dt=0) == UNSUPPORTED                    # bf16 only, like the backward
    assert pb(Dk=96) == UNSUPPORTED
    assert pb(A=None) == NULL
    assert pb(dA=None) == NULL
    assert pb(qr=None) == NULL
    assert pb(N=2, B=1) == SHAPE
    assert pb(cu=P, B=2, N=2) == SHAPE
    assert pb(qr=ctypes.c_void_p(0x1008)) == UNSUPPORTED  # rows must be 16-byte aligned
    assert pb(wsb=need - 1) == WORKSPACE
    assert pb(ws=None) == WORKSPACE
    assert pb(ws=ctypes.c_void_p(0x1010)) == WORKSPACE


def test_short_conv_bwd_validation():
    L = kda.lib()
    need = L.kda_short_conv_bwd_workspace_bytes(1, 300, 16, 4)
    assert need >= 2 * 4 * 16 * 4                     # two 256-token runs of W x C fp32 partials
    assert L.kda_short_conv_bwd_workspace_bytes(1, 300, 12, 4) == 0

    def cb(x=P, w=P, dy=P, dw=P, dt=1, W=4, C=16, ws=P, wsb=need, N=1, B=1, T=300, cu=None):
        return L.kda_short_conv_bwd(x, w, None, dy, None, P, dw, None, cu, N, B, T, C, W, dt, ws, wsb, None)

    assert cb(dt=7) == DTYPE
    assert cb(W=9) == UNSUPPORTED
    assert cb(C=12) == UNSUPPORTED
    assert cb(dw=None) == NULL
    assert cb(dy=None) == NULL
    assert cb(N=2) == SHAPE
    assert cb(x=ctypes.c_void_p(0x1008)) == UNSUPPORTED
    assert cb(wsb=need - 1) == WORKSPACE
    assert cb(ws=None) == WORKSPACE
