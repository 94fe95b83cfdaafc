"""CPU fp64 oracle for the fused gate and normalisation prologue of KDA.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use it.  It shares no code with the HIP path.

What it computes
----------------
The steps that turn a layer's raw projections into the KDA inputs the
recurrence uses:

* q and k are L2-normalised per token and head (the configurations draw
  "L2-normalised per token" queries and keys).
* The Kimi-K3-Tiny-L13 card names KDA's A_log and dt_bias as real
  parameters, and the Mini-K3-1H-mamba2 README lists A_log and dt_bias as
  Mamba-style state controls.  The pages give no gate formula.  The reading
  here is the Mamba-style one:
      g = -exp(A_log) * softplus(f + dt_bias)
  per key channel (or per 64-channel decay group), with softplus(x) =
  log(1 + e^x).  So alpha = e^g lies in (0, 1).
* beta = sigmoid(b) per token and head.

The normalisation carries a guard eps = 1e-6 inside the square root:
x / sqrt(sum x^2 + eps).  For unit rows this changes them by under 1e-6.

The result is exactly kda_oracle.kda_forward (or kda_decode_step) applied to
the prepared inputs.

Backward (the miniKimiK3 card's KDA bullet: KDA trains through the chunked
form; the prologue's parameters A_log and dt_bias are trained with it).  The
reverse mode of each step above, written from its definition:

* y = x r with r = (sum x^2 + eps)^(-1/2):  dx = r (dy - y (y . dy));
* g = -exp(A_log) softplus(f + dt_bias):  dg/df = dg/d(dt_bias)
  = -exp(A_log) sigmoid(f + dt_bias), dg/d(A_log) = g; A_log and dt_bias are
  shared by every token, so their gradients sum over tokens (and sequences);
* beta = sigmoid(b):  d beta / db = beta (1 - beta).
"""

import numpy as np

from .kda_backward import kda_backward
from .kda_oracle import kda_decode_step, kda_decode_step_pool, kda_forward

EPS = 1e-6

__all__ = ["EPS", "l2_normalize", "softplus", "sigmoid", "gate", "prepare", "kda_forward_prologue",
           "kda_decode_step_prologue", "kda_decode_step_pool_prologue", "l2_normalize_backward",
           "prologue_backward", "kda_backward_prologue"]


def l2_normalize(x, eps=EPS):
    """x / sqrt(sum over the last axis of x^2 + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def softplus(x):
    """log(1 + e^x), computed without overflow as logaddexp(0, x)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def gate(f, A_log, dt_bias):
    """g = -exp(A_log) * softplus(f + dt_bias); A_log and dt_bias broadcast
    over the leading (token) axes: [H, dk // g_group]."""
    f = np.asarray(f, dtype=np.float64)
    return -np.exp(np.asarray(A_log, dtype=np.float64)) * softplus(f + np.asarray(dt_bias, dtype=np.float64))


def prepare(q_raw, k_raw, f, b_raw, A_log, dt_bias):
    """The prologue on its own: returns (q, k, g, beta)."""
    return l2_normalize(q_raw), l2_normalize(k_raw), gate(f, A_log, dt_bias), sigmoid(b_raw)


def kda_forward_prologue(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, h0=None, cu_seqlens=None, g_group=1):
    """The prologue followed by the chunked-form forward (same result as the
    sequential recurrence).  Shapes as kda_forward with f in place of g and
    b_raw in place of beta; A_log, dt_bias [H, dk // g_group]."""
    q, k, g, beta = prepare(q_raw, k_raw, f, b_raw, A_log, dt_bias)
    return kda_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu_seqlens, g_group=g_group)


def kda_decode_step_prologue(state, q_raw, k_raw, v, f, b_raw, A_log, dt_bias, g_group=1):
    """The prologue followed by one decode step ([N, H, ...] inputs)."""
    q, k, g, beta = prepare(q_raw, k_raw, f, b_raw, A_log, dt_bias)
    return kda_decode_step(state, q, k, v, g, beta, g_group=g_group)


def kda_decode_step_pool_prologue(pool, slots, q_raw, k_raw, v, f, b_raw, A_log, dt_bias, g_group=1,
                                  state_dtype=None, o_gate=None):
    """The prologue followed by one serving-pool decode step (see
    kda_decode_step_pool for the slots, the state dtype and the output gate)."""
    q, k, g, beta = prepare(q_raw, k_raw, f, b_raw, A_log, dt_bias)
    return kda_decode_step_pool(pool, slots, q, k, v, g, beta, g_group=g_group, state_dtype=state_dtype,
                                o_gate=o_gate)


def l2_normalize_backward(x, dy, eps=EPS):
    """Gradient of l2_normalize(x) against the cotangent dy (last axis):
    r (dy - y (y . dy)) with y = x r, r = (sum x^2 + eps)^(-1/2)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    return r * (dy - y * np.sum(y * dy, axis=-1, keepdims=True))


def prologue_backward(q_raw, k_raw, f, b_raw, A_log, dt_bias, dq, dk, dg, dbeta):
    """Gradients of the prologue's inputs from those of its outputs (q, k,
    g, beta as prepare returns them).  f, dg: [..., H, dk // g_group];
    A_log, dt_bias: [H, dk // g_group].  Returns a dict of dq_raw, dk_raw,
    df, db_raw, dA_log, ddt_bias; the last two are summed over every
    leading (batch, token) axis."""
    f = np.asarray(f, dtype=np.float64)
    A = np.asarray(A_log, dtype=np.float64)
    bias = np.asarray(dt_bias, dtype=np.float64)
    dg = np.asarray(dg, dtype=np.float64)
    g = gate(f, A, bias)
    dfb = dg * (-np.exp(A) * sigmoid(f + bias))
    lead = tuple(range(f.ndim - 2))
    beta = sigmoid(b_raw)
    return {
        "dq_raw": l2_normalize_backward(q_raw, dq),
        "dk_raw": l2_normalize_backward(k_raw, dk),
        "df": dfb,
        "db_raw": np.asarray(dbeta, dtype=np.float64) * beta * (1.0 - beta),
        "dA_log": np.sum(dg * g, axis=lead),
        "ddt_bias": np.sum(dfb, axis=lead),
    }


def kda_backward_prologue(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, do, h0=None, dht=None, cu_seqlens=None,
                          g_group=1):
    """Gradients of L = <do, o> + <dht, ht> for kda_forward_prologue with
    respect to q_raw, k_raw, v, f, b_raw, A_log, dt_bias and h0: the plain
    backward on the prepared inputs, then prologue_backward."""
    q, k, g, beta = prepare(q_raw, k_raw, f, b_raw, A_log, dt_bias)
    gr = kda_backward(q, k, v, g, beta, do, h0=h0, dht=dht, cu_seqlens=cu_seqlens, g_group=g_group)
    out = prologue_backward(q_raw, k_raw, f, b_raw, A_log, dt_bias, gr["dq"], gr["dk"], gr["dg"], gr["dbeta"])
    out["dv"] = gr["dv"]
    out["dh0"] = gr["dh0"]
    return out
