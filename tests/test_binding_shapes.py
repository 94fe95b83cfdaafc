"""The Python binding checks every tensor's full shape against the sizes it
derives from q (or x) before any library call, and raises ValueError on a
mismatch: the kernels size every access from those sizes, so a smaller
state, output or gradient tensor would be written out of bounds on the
device.  CPU tensors suffice, because the shape checks run first."""

import pytest
import torch

from gated_delta_rule_04_amd import kda

B, T, H, DK, DV = 2, 8, 3, 64, 64
N = B


def _pre(dt=torch.bfloat16, gg=1):
    z = lambda *s: torch.zeros(*s, dtype=dt)
    return dict(q=z(B, T, H, DK), k=z(B, T, H, DK), v=z(B, T, H, DV), g=z(B, T, H, DK // gg), beta=z(B, T, H))


def _dec(dt=torch.bfloat16):
    z = lambda *s: torch.zeros(*s, dtype=dt)
    return dict(q=z(N, H, DK), k=z(N, H, DK), v=z(N, H, DV), g=z(N, H, DK), beta=z(N, H))


def _shape_error(fn, *a, **kw):
    with pytest.raises(ValueError, match=r"must have shape|must be \[|must be [34]-d"):
        fn(*a, **kw)


@pytest.mark.parametrize("name,bad", [("k", (B, T, H, DK - 1)), ("v", (B, T + 1, H, DV)), ("g", (B, T, H + 1, DK)),
                                      ("beta", (B, T, H, 1)), ("beta", (B, T))])
def test_chunk_fwd_inputs(name, bad):
    d = _pre()
    d[name] = torch.zeros(*bad, dtype=torch.bfloat16)
    _shape_error(kda.chunk_fwd, **d)


@pytest.mark.parametrize("kw,shape", [("initial_state", (N, H, DK, DV - 1)), ("initial_state", (N - 1, H, DK, DV)),
                                      ("final_state", (N, H, DK - 1, DV)), ("out", (B, T, H, DV // 2))])
def test_chunk_fwd_states_and_out(kw, shape):
    d = _pre()
    dt = torch.bfloat16 if kw == "out" else torch.float32
    _shape_error(kda.chunk_fwd, **d, **{kw: torch.zeros(*shape, dtype=dt)})


def test_chunk_fwd_packed_needs_one_row():
    d = _pre()
    cu = torch.tensor([0, 4, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="B == 1"):
        kda.chunk_fwd(**d, cu_seqlens=cu)


def test_chunk_fwd_prologue_shapes():
    d = _pre()
    A = torch.zeros(H, DK)
    dtb = torch.zeros(H, DK)
    _shape_error(kda.chunk_fwd_prologue, d["q"], d["k"], d["v"], d["g"], d["beta"], A, dtb,
                 initial_state=torch.zeros(N, H, DK, DV + 1))
    _shape_error(kda.chunk_fwd_prologue, d["q"], d["k"][:, :-1], d["v"], d["g"], d["beta"], A, dtb)


def test_chunk_fwd_save_shapes():
    d = _pre()
    _shape_error(kda.chunk_fwd_save, **d, final_state=torch.zeros(N, H, DK, DV - 1))


@pytest.mark.parametrize("name", ["dq", "dk", "dv", "dg", "dbeta", "dh0"])
def test_chunk_bwd_outputs(name):
    d = _pre()
    do = torch.zeros(B, T, H, DV, dtype=torch.bfloat16)
    shapes = {"dq": (B, T, H, DK - 8), "dk": (B, T - 1, H, DK), "dv": (B, T, H, 1), "dg": (B, T, H, DK // 2),
              "dbeta": (B, T, H, 1), "dh0": (N, H, DK, DV - 1)}
    dt = torch.float32 if name == "dh0" else torch.bfloat16
    _shape_error(kda.chunk_bwd, **d, do=do, out={name: torch.zeros(*shapes[name], dtype=dt)})


def test_chunk_bwd_cotangents():
    d = _pre()
    _shape_error(kda.chunk_bwd, **d, do=torch.zeros(B, T, H, DV - 1, dtype=torch.bfloat16))
    _shape_error(kda.chunk_bwd, **d, do=torch.zeros(B, T, H, DV, dtype=torch.bfloat16),
                 dht=torch.zeros(N, H, DK, DV // 2))


@pytest.mark.parametrize("name,bad", [("k", (N, H, DK + 1)), ("v", (N + 1, H, DV)), ("g", (N, H - 1, DK)),
                                      ("beta", (N,))])
def test_recurrent_step_inputs(name, bad):
    d = _dec()
    d[name] = torch.zeros(*bad, dtype=torch.bfloat16)
    _shape_error(kda.recurrent_step, **d, state=torch.zeros(N, H, DK, DV))


def test_recurrent_step_state_and_out():
    d = _dec()
    _shape_error(kda.recurrent_step, **d, state=torch.zeros(N, H, DK, DV - 1))
    _shape_error(kda.recurrent_step, **d, state=torch.zeros(N - 1, H, DK, DV))
    _shape_error(kda.recurrent_step, **d, state=torch.zeros(N, H, DK, DV),
                 out=torch.zeros(N, H, DV - 1, dtype=torch.bfloat16))


def test_recurrent_step_prologue_shapes():
    d = _dec()
    A = torch.zeros(H, DK)
    _shape_error(kda.recurrent_step_prologue, d["q"], d["k"], d["v"], d["g"], d["beta"], A, A.clone(),
                 torch.zeros(N, H, DK // 2, DV))


def test_recurrent_step_pool_shapes():
    d = _dec()
    pool = torch.zeros(5, H, DK, DV)
    slots = torch.zeros(N, dtype=torch.int32)
    _shape_error(kda.recurrent_step_pool, d["q"], d["k"], d["v"], d["g"], d["beta"][:, :1], pool, slots)
    _shape_error(kda.recurrent_step_pool, d["q"], d["k"], d["v"], d["g"], d["beta"], pool, slots,
                 out=torch.zeros(N, H, 1, dtype=torch.bfloat16))
    A = torch.zeros(H, DK)
    _shape_error(kda.recurrent_step_pool_prologue, d["q"], d["k"][:1], d["v"], d["g"], d["beta"], A, A.clone(),
                 pool, slots)


def test_short_conv_shapes():
    x = torch.zeros(B, T, 16, dtype=torch.bfloat16)
    w = torch.zeros(16, 4, dtype=torch.bfloat16)
    _shape_error(kda.short_conv_fwd, x, w, conv0=torch.zeros(N, 2, 16, dtype=torch.bfloat16))
    _shape_error(kda.short_conv_fwd, x, w, out=torch.zeros(B, T, 8, dtype=torch.bfloat16))
    _shape_error(kda.short_conv_fwd, x, torch.zeros(8, 4, dtype=torch.bfloat16))
    xs = torch.zeros(N, 16, dtype=torch.bfloat16)
    _shape_error(kda.short_conv_step, xs, w, torch.zeros(N, 3, 8, dtype=torch.bfloat16))
    _shape_error(kda.short_conv_step, xs, w, torch.zeros(N, 3, 16, dtype=torch.bfloat16),
                 out=torch.zeros(N, 8, dtype=torch.bfloat16))


@pytest.mark.parametrize("name,shape", [("dq_raw", (B, T, H, DK - 1)), ("dv", (B, T + 1, H, DV)),
                                        ("dA_log", (H, DK + 1)), ("dh0", (N, H, DK, DV - 1))])
def test_chunk_bwd_prologue_out_shapes(name, shape):
    """Preallocated gradient buffers are checked like every other tensor."""
    d = _pre()
    A = torch.zeros(H, DK)
    dt = torch.float32 if name in ("dA_log", "dh0") else torch.bfloat16
    _shape_error(kda.chunk_bwd_prologue, d["q"], d["k"], d["v"], d["g"], d["beta"], A, A.clone(),
                 torch.zeros(B, T, H, DV, dtype=torch.bfloat16), out={name: torch.zeros(*shape, dtype=dt)})


def test_chunk_bwd_prologue_out_names_and_types():
    d = _pre()
    A = torch.zeros(H, DK)
    do = torch.zeros(B, T, H, DV, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="unknown gradient"):
        kda.chunk_bwd_prologue(d["q"], d["k"], d["v"], d["g"], d["beta"], A, A.clone(), do,
                               out={"dq": torch.zeros(B, T, H, DK, dtype=torch.bfloat16)})
    with pytest.raises(TypeError, match="dh0 must be"):
        kda.chunk_bwd_prologue(d["q"], d["k"], d["v"], d["g"], d["beta"], A, A.clone(), do,
                               out={"dh0": torch.zeros(N, H, DK, DV, dtype=torch.bfloat16)})
