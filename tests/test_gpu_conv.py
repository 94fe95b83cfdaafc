"""Short causal convolution on the GPU (through the C-ABI) against the CPU
oracle: widths, dtypes, packed documents, initial and final conv states,
split equivalence and the decode step."""

import numpy as np
import pytest
import torch

from gated_delta_rule_04_amd import kda
from oracle.short_conv import short_conv_forward, short_conv_step
from tests._parity import assert_close

pytestmark = pytest.mark.gpu


def _t(a, dt):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(dt)


def _draw(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("B,T,C", [(2, 300, 64), (1, 129, 8), (3, 64, 200)])
def test_conv_fwd_batch(dt, W, B, T, C):
    seed = W * 100 + T + C
    x, w = _t(_draw((B, T, C), seed), dt), _t(_draw((C, W), seed + 1, 0.5), dt)
    c0 = _t(_draw((B, W - 1, C), seed + 2), dt)
    y, f = kda.short_conv_fwd(x.cuda(), w.cuda(), conv0=c0.cuda(), output_final_state=True)
    yr, fr = short_conv_forward(x.float(), w.float(), conv0=c0.float())
    torch.cuda.synchronize()
    assert_close("conv y W=%d" % W, y.cpu(), yr, dt)
    assert torch.equal(f.cpu(), torch.from_numpy(fr).to(dt))  # the final state is a copy of inputs


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_conv_fwd_varlen_short_and_empty_documents(dt):
    C, W = 96, 4
    cu = np.array([0, 2, 2, 70, 71, 200, 203, 333], dtype=np.int32)  # lengths 2, 0, 68, 1, 129, 3, 130
    T = int(cu[-1])
    x, w = _t(_draw((1, T, C), 21), dt), _t(_draw((C, W), 22, 0.5), dt)
    N = len(cu) - 1
    for with_c0 in (False, True):
        c0 = _t(_draw((N, W - 1, C), 23), dt) if with_c0 else None
        y, f = kda.short_conv_fwd(x.cuda(), w.cuda(), conv0=None if c0 is None else c0.cuda(),
                                  output_final_state=True, cu_seqlens=torch.from_numpy(cu).cuda())
        yr, fr = short_conv_forward(x.float(), w.float(), conv0=None if c0 is None else c0.float(), cu_seqlens=cu)
        torch.cuda.synchronize()
        assert_close("conv varlen y c0=%s" % with_c0, y.cpu(), yr, dt)
        assert torch.equal(f.cpu(), torch.from_numpy(fr).to(dt))


def test_conv_split_equivalence_bitwise():
    dt, C, W = torch.bfloat16, 128, 4
    x, w = _t(_draw((2, 400, C), 31), dt).cuda(), _t(_draw((C, W), 32, 0.5), dt).cuda()
    y, f = kda.short_conv_fwd(x, w, output_final_state=True)
    ya, fa = kda.short_conv_fwd(x[:, :191].contiguous(), w, output_final_state=True)
    yb, fb = kda.short_conv_fwd(x[:, 191:].contiguous(), w, conv0=fa, output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([ya, yb], dim=1), y) and torch.equal(fb, f)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("W", [1, 3, 4])
def test_conv_decode_steps_match_oracle_and_forward(dt, W):
    N, C, steps = 5, 72, 9
    w = _t(_draw((C, W), 41 + W, 0.5), dt)
    st0 = _t(_draw((N, W - 1, C), 42), dt)
    xs = _t(_draw((N, steps, C), 43), dt)
    st = st0.clone().cuda()
    ref = st0.float().numpy()
    for s in range(steps):
        y = kda.short_conv_step(xs[:, s].contiguous().cuda(), w.cuda(), st if W > 1 else None)
        yr, ref = short_conv_step(xs[:, s].float(), w.float(), ref)
        ref = torch.from_numpy(ref).to(dt).float().numpy()  # the state holds inputs: exact in dt
        torch.cuda.synchronize()
        assert_close("conv step %d W=%d" % (s, W), y.cpu(), yr, dt)
    yf, ff = short_conv_forward(xs.float(), w.float(), conv0=st0.float())
    assert torch.equal(st.cpu(), torch.from_numpy(ff).to(dt)) if W > 1 else True


def test_conv_k3_projection_width_sampled():
    """The width of one K3 projection (96 heads x 128 = 12288 channels) over
    32768 tokens, W = 4; oracle on sampled channels."""
    dt, B, T, C, W = torch.bfloat16, 1, 32768, 12288, 4
    g = torch.Generator().manual_seed(51)
    x = torch.randn((B, T, C), generator=g).to(dt)
    w = (0.5 * torch.randn((C, W), generator=g)).to(dt)
    y, _ = kda.short_conv_fwd(x.cuda(), w.cuda())
    torch.cuda.synchronize()
    ch = np.array([0, 7, 8, 5000, 12287])
    yr, _ = short_conv_forward(x[:, :, ch].float(), w[ch].float())
    assert_close("conv k3 sampled", y.cpu()[:, :, ch], yr, dt)


# ---------------------------------------------------------------- backward
from oracle.short_conv import short_conv_backward  # noqa: E402


def _conv_bwd_check(tag, got, ref, dt):
    dx, dw, dc0 = ref
    assert_close(tag + " dx", got["dx"].cpu(), dx, dt)
    # dweight is an fp32 sum over every token: compared relative to its scale
    gw = got["dweight"].cpu().double().numpy()
    assert np.max(np.abs(gw - dw)) <= 1e-5 * max(1.0, np.max(np.abs(dw))), tag + " dweight"
    if dc0.size:
        assert_close(tag + " dconv0", got["dconv0"].cpu(), dc0, dt)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("B,T,C", [(2, 300, 64), (1, 129, 8), (3, 64, 200)])
def test_conv_bwd_batch(dt, W, B, T, C):
    seed = 1000 + W * 100 + T + C
    x, w = _t(_draw((B, T, C), seed), dt), _t(_draw((C, W), seed + 1, 0.5), dt)
    c0 = _t(_draw((B, W - 1, C), seed + 2), dt)
    dy = _t(_draw((B, T, C), seed + 3), dt)
    dfin = _t(_draw((B, W - 1, C), seed + 4), dt)
    got = kda.short_conv_bwd(x.cuda(), w.cuda(), dy.cuda(), conv0=c0.cuda(), dconv_final=dfin.cuda())
    torch.cuda.synchronize()
    ref = short_conv_backward(x.float(), w.float(), dy.float(), conv0=c0.float(), dfinal=dfin.float())
    _conv_bwd_check("conv bwd W=%d B%d T%d C%d" % (W, B, T, C), got, ref, dt)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_conv_bwd_varlen_short_and_empty_documents(dt):
    C, W = 96, 4
    cu = np.array([0, 2, 2, 70, 71, 200, 203, 333, 590], dtype=np.int32)  # 2, 0, 68, 1, 129, 3, 130, 257
    T, N = int(cu[-1]), len(cu) - 1
    x, w = _t(_draw((1, T, C), 41), dt), _t(_draw((C, W), 42, 0.5), dt)
    dy = _t(_draw((1, T, C), 43), dt)
    for with_states in (False, True):
        c0 = _t(_draw((N, W - 1, C), 44), dt) if with_states else None
        dfin = _t(_draw((N, W - 1, C), 45), dt) if with_states else None
        got = kda.short_conv_bwd(x.cuda(), w.cuda(), dy.cuda(), conv0=None if c0 is None else c0.cuda(),
                                 dconv_final=None if dfin is None else dfin.cuda(),
                                 cu_seqlens=torch.from_numpy(cu).cuda())
        torch.cuda.synchronize()
        ref = short_conv_backward(x.float(), w.float(), dy.float(), conv0=None if c0 is None else c0.float(),
                                  dfinal=None if dfin is None else dfin.float(), cu_seqlens=cu)
        _conv_bwd_check("conv bwd varlen states=%s" % with_states, got, ref, dt)


def test_conv_bwd_k3_width_sampled_channels_and_deterministic():
    """One K3 projection width (12,288 channels) over 32,768 tokens, W = 4,
    bf16: channels are independent, so the oracle on three groups of 8
    channels (both ends and the middle) checks the full-size launch; two
    calls give the same bits."""
    dt, B, T, C, W = torch.bfloat16, 1, 32768, 12288, 4
    g = torch.Generator().manual_seed(51)
    x = torch.randn((B, T, C), generator=g).to(dt).cuda()
    w = (0.5 * torch.randn((C, W), generator=g)).to(dt).cuda()
    dy = torch.randn((B, T, C), generator=g).to(dt).cuda()
    a = kda.short_conv_bwd(x, w, dy)
    b = kda.short_conv_bwd(x, w, dy)
    torch.cuda.synchronize()
    for n in ("dx", "dweight"):
        assert torch.equal(a[n], b[n]), n
    sel = np.r_[0:8, 6144:6152, C - 8:C]
    xs, ws, dys = (t.cpu()[..., sel] if t.dim() == 3 else t.cpu()[sel] for t in (x, w, dy))
    ref = short_conv_backward(xs.float(), ws.float(), dys.float())
    got = {"dx": a["dx"][..., sel], "dweight": a["dweight"][sel], "dconv0": a["dconv0"][..., sel]}
    _conv_bwd_check("conv bwd K3 width", got, ref, dt)
