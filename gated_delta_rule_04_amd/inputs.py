"""Seeded synthetic inputs for the KDA workloads.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle's tests: it draws random inputs and nothing else.  It holds none of the
method's arithmetic (no decay, no state update, no read-out).

Recipe (the same for every workload; shapes come from the pages):

* All draws are float64 from ``numpy.random.default_rng(seed)``, in this
  order: q, k, v, beta-logit, g-logit, [initial state], then the per-step
  draws of a decode run (q, k, v, beta-logit, g-logit per step).
* q, k: z ~ N(0, 1)^dk, divided by its L2 norm per (token, head).
* v: N(0, 1).
* beta = sigmoid(z).
* g = log(alpha) = -softplus(z - shift) with shift = 2 ("config" decay,
  alpha ~ (0.3, 1)), 6 ("slow" decay, alpha ~ 0.998), or g = 0 ("none").
  With g_group = 64 one value is drawn per (token, head, 64-channel group).
* Initial decode states: N(0, 0.02^2) (0.02 read as the standard deviation).
* The float64 values are rounded to float32 (round-to-nearest-even) and, for
  bf16 workloads, then to bfloat16 (round-to-nearest-even).  Both the GPU and
  the oracle consume exactly these rounded values.
* Packed-document lengths: L ~ Geometric(p = 1/1500) on {1, 2, ...}, clipped
  to [16, 8192], drawn from ``default_rng(len_seed)`` until the sum reaches
  the packed length; the last length is cut to fill exactly, and merged into
  the previous document when the cut leaves fewer than 16 tokens.
"""

import hashlib

import numpy as np
import torch

__all__ = [
    "WORKLOADS",
    "doc_lengths",
    "make_prefill",
    "make_decode",
    "workload_prefill",
    "workload_decode",
    "sha256_of",
]

# The five workloads.  Shapes: miniKimiK3 (8 heads x 64, 8,192 tokens per
# step), Mini-K3-1H (12 heads x 128, 8K rows x B5, decay-g64 ablation),
# packed documents, and Kimi-K3 (96 KDA heads x 128; decode batches beyond 43).
WORKLOADS = {
    "tiny_f32": dict(kind="prefill", B=1, T=256, H=1, dk=64, dv=64, dtype="f32", g_group=1, seed=1000),
    "minikimi_bf16": dict(kind="prefill", B=16, T=512, H=8, dk=64, dv=64, dtype="bf16", g_group=1, seed=1001),
    "mini1h_g64_bf16": dict(kind="prefill", B=5, T=8192, H=12, dk=128, dv=128, dtype="bf16", g_group=64, seed=1002),
    "varlen_bf16": dict(kind="prefill", B=1, T=65536, H=12, dk=128, dv=128, dtype="bf16", g_group=1, seed=1003,
                        varlen=True, len_seed=2003),
    "k3_prefill_bf16": dict(kind="prefill", B=1, T=32768, H=96, dk=128, dv=128, dtype="bf16", g_group=1, seed=1004),
    "k3_decode_bf16": dict(kind="decode", N=256, H=96, dk=128, dv=128, dtype="bf16", g_group=1, steps=64,
                           seed=1104, state_std=0.02),
}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_BLOCK_ELEMS = 1 << 24  # rows are drawn in blocks of about this many values


def sha256_of(t):
    """sha256 of a tensor's raw bytes (CPU tensor or numpy array)."""
    if isinstance(t, torch.Tensor):
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        t = t.numpy()
    return hashlib.sha256(np.ascontiguousarray(t).tobytes()).hexdigest()


def _round_to(x64, dtype):
    """float64 -> float32 (RNE) -> target dtype (RNE for bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return t.to(_TORCH_DTYPE[dtype])


def _unit_rows(z):
    return z / np.linalg.norm(z, axis=-1, keepdims=True)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _neg_softplus_shift(shift):
    return lambda z: -np.logaddexp(0.0, z - shift)


def _draw(rng, shape, dtype, fn=None):
    """Draw N(0,1) of `shape` row-block by row-block (same stream as one draw),
    apply `fn` to each block in float64, round to `dtype`."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=_TORCH_DTYPE[dtype])
    if len(shape) == 0 or out.numel() == 0:
        return out
    rows = shape[0]
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    step = max(1, _BLOCK_ELEMS // max(per_row, 1))
    flat = out.view(rows, -1) if len(shape) > 1 else out.view(rows, 1)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = rng.standard_normal((r1 - r0,) + shape[1:])
        if fn is not None:
            z = fn(z)
        flat[r0:r1] = _round_to(z, dtype).reshape(r1 - r0, -1)
    return out


def _decay_fn(decay):
    if decay == "config":
        return _neg_softplus_shift(2.0)
    if decay == "slow":
        return _neg_softplus_shift(6.0)
    if decay == "none":
        return lambda z: np.zeros_like(z)
    if decay.startswith("strong:"):
        # "strong:S": every third key channel (or decay group) decays by about
        # e^S over 64 tokens, g = (S / 64) (1 + 0.2 tanh z) per token; the
        # others as "config"
        per_token = float(decay.split(":", 1)[1]) / 64.0
        cfg = _neg_softplus_shift(2.0)

        def fn(z):
            out = cfg(z)
            out[..., ::3] = per_token * (1.0 + 0.2 * np.tanh(z[..., ::3]))
            return out
        return fn
    raise ValueError("unknown decay recipe %r" % (decay,))


def doc_lengths(total, len_seed, mean=1500, lo=16, hi=8192):
    """Packed-document lengths summing exactly to `total` (see module doc)."""
    rng = np.random.default_rng(len_seed)
    lens = []
    acc = 0
    while acc < total:
        L = int(np.clip(rng.geometric(1.0 / mean), lo, hi))
        lens.append(L)
        acc += L
    lens[-1] -= acc - total
    if lens[-1] < lo and len(lens) > 1:
        last = lens.pop()
        lens[-1] += last
    return lens


def make_prefill(B, T, H, dk, dv, dtype="bf16", g_group=1, seed=0, decay="config",
                 h0=False, cu_seqlens=None, state_std=0.02):
    """Synthetic prefill inputs.  Returns a dict of CPU torch tensors:
    q, k [B,T,H,dk]; v [B,T,H,dv]; g [B,T,H,dk//g_group]; beta [B,T,H]
    (all in `dtype`), h0 [N,H,dk,dv] float32 or None, cu_seqlens int32 or None."""
    if dk % g_group:
        raise ValueError("g_group must divide dk")
    rng = np.random.default_rng(seed)
    rows = B * T
    q = _draw(rng, (rows, H, dk), dtype, _unit_rows).view(B, T, H, dk)
    k = _draw(rng, (rows, H, dk), dtype, _unit_rows).view(B, T, H, dk)
    v = _draw(rng, (rows, H, dv), dtype).view(B, T, H, dv)
    beta = _draw(rng, (rows, H), dtype, _sigmoid).view(B, T, H)
    g = _draw(rng, (rows, H, dk // g_group), dtype, _decay_fn(decay)).view(B, T, H, dk // g_group)
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = torch.as_tensor(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.numel() - 1
    h0_t = None
    if h0:
        h0_t = _draw(rng, (N, H, dk, dv), "f32", lambda z: state_std * z)
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0_t, cu_seqlens=cu, g_group=g_group)


def make_prologue(B, T, H, dk, dv, dtype="bf16", g_group=1, seed=0, h0=False, cu_seqlens=None, state_std=0.02,
                  qk_scale=(0.25, 8.0), a_log_mean=0.0):
    """Raw inputs of the fused gate/normalisation prologue.  q_raw, k_raw
    [B,T,H,dk]: N(0,1) rows times a per-row scale drawn log-uniformly from
    qk_scale (not normalised); v [B,T,H,dv] N(0,1); gate logits f
    [B,T,H,dk//g_group] N(0,1); beta logits b_raw [B,T,H] N(0,1); A_log,
    dt_bias [H, dk//g_group] float32 ~ N(0, 0.1^2) and N(-2, 0.1^2), so that
    the gate reproduces the -softplus(z - 2) decay of the other workloads;
    a_log_mean shifts A_log (ln 16: a Mamba-style A of about 16, per-token
    log-decays near -2 and summed over 64 tokens near -130)."""
    rng = np.random.default_rng(seed)
    rows = B * T
    lo, hi = np.log(qk_scale[0]), np.log(qk_scale[1])
    scaled = lambda z: z * np.exp(rng.uniform(lo, hi, z.shape[:-1] + (1,)))
    q = _draw(rng, (rows, H, dk), dtype, scaled).view(B, T, H, dk)
    k = _draw(rng, (rows, H, dk), dtype, scaled).view(B, T, H, dk)
    v = _draw(rng, (rows, H, dv), dtype).view(B, T, H, dv)
    b = _draw(rng, (rows, H), dtype).view(B, T, H)
    f = _draw(rng, (rows, H, dk // g_group), dtype).view(B, T, H, dk // g_group)
    A_log = torch.as_tensor(a_log_mean + 0.1 * rng.standard_normal((H, dk // g_group)), dtype=torch.float32)
    dt_bias = torch.as_tensor(-2.0 + 0.1 * rng.standard_normal((H, dk // g_group)), dtype=torch.float32)
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = torch.as_tensor(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.numel() - 1
    h0_t = _draw(rng, (N, H, dk, dv), "f32", lambda z: state_std * z) if h0 else None
    return dict(q_raw=q, k_raw=k, v=v, f=f, b_raw=b, A_log=A_log, dt_bias=dt_bias, h0=h0_t, cu_seqlens=cu,
                g_group=g_group)


def make_cotangents(B, T, H, dk, dv, N, dtype="bf16", seed=0, state_std=0.02, final_state=True):
    """Synthetic output cotangents for a backward pass: do [B,T,H,dv] ~ N(0, 1)
    in `dtype` and, if final_state, dht [N,H,dk,dv] float32 ~ N(0, state_std^2)."""
    rng = np.random.default_rng(seed)
    do = _draw(rng, (B * T, H, dv), dtype).view(B, T, H, dv)
    dht = _draw(rng, (N, H, dk, dv), "f32", lambda z: state_std * z) if final_state else None
    return dict(do=do, dht=dht)


def make_decode(N, H, dk, dv, steps, dtype="bf16", g_group=1, seed=0, state_std=0.02, decay="config"):
    """Synthetic decode run: initial fp32 state [N,H,dk,dv] ~ N(0, state_std^2)
    and `steps` per-step input dicts (q, k [N,H,dk]; v [N,H,dv]; g; beta)."""
    rng = np.random.default_rng(seed)
    state = _draw(rng, (N, H, dk, dv), "f32", lambda z: state_std * z)
    per_step = []
    for _ in range(steps):
        q = _draw(rng, (N, H, dk), dtype, _unit_rows)
        k = _draw(rng, (N, H, dk), dtype, _unit_rows)
        v = _draw(rng, (N, H, dv), dtype)
        beta = _draw(rng, (N, H), dtype, _sigmoid)
        g = _draw(rng, (N, H, dk // g_group), dtype, _decay_fn(decay))
        per_step.append(dict(q=q, k=k, v=v, g=g, beta=beta))
    return dict(state=state, steps=per_step, g_group=g_group)


def workload_prefill(name):
    """Inputs of a named prefill workload (see WORKLOADS)."""
    w = WORKLOADS[name]
    if w["kind"] != "prefill":
        raise ValueError(name + " is not a prefill workload")
    cu = None
    if w.get("varlen"):
        lens = doc_lengths(w["T"], w["len_seed"])
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return make_prefill(w["B"], w["T"], w["H"], w["dk"], w["dv"], w["dtype"], w["g_group"], w["seed"],
                        cu_seqlens=cu)


def workload_decode(name, steps=None):
    """Inputs of a named decode workload (see WORKLOADS)."""
    w = WORKLOADS[name]
    if w["kind"] != "decode":
        raise ValueError(name + " is not a decode workload")
    return make_decode(w["N"], w["H"], w["dk"], w["dv"], w["steps"] if steps is None else steps,
                       w["dtype"], w["g_group"], w["seed"], w["state_std"])
