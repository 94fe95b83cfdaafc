"""CPU fp64 oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
routes through it and shares no code with it.

What it computes
----------------
The plain sequential KDA recurrence, one token at a time, in float64, on the
float64 up-cast of the exact input values the GPU receives.

Sources (the page text the method is defined on):

* miniKimiK3 model card, section "Architecture", the Kimi Delta Attention
  bullet: the state update is one gradient-descent step on the squared error
  of the state's read-out against v, with per-channel gated decay; a chunked
  parallel form for training and a fixed-size recurrence for decoding.
* The matrix form of that bullet: S_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
  S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.
* Mini-K3-1H-mamba2 README excerpt (packed-document paragraph): packed
  documents are causally isolated and recurrent state flow is reset at every
  document boundary.
* Mini-K3-1H-decay-g64 model card: decay granularity ("decay-g64") is an
  ablation axis -- one log-decay value shared by a group of 64 channels.

Readings where the pages are silent:

* The gradient step is on 1/2 ||S^T k - v||^2 with step size beta; this gives
  exactly the matrix form above (a literal ||.||^2 would double the step).
* Decay is applied first, then the delta write, and it scales the key-channel
  axis (rows of S, length d_k).
* o_t reads the state after the token's own write.
* No query scale, no in-kernel normalisation, no gate activation: q, k, v,
  g = log(alpha) <= 0 and beta arrive ready to use.
* With cu_seqlens each document starts from h0[doc] (zeros if absent) and
  returns its own final state; a zero-length document returns h0[doc].
* The serving pool's output gate (the Mini-K3-1H cards list output gates
  without a formula) is the elementwise logistic gate o * sigmoid(z) on the
  step's output; it never reaches the state.

Layouts follow the library: q, k [B, T, H, dk]; v [B, T, H, dv];
g [B, T, H, dk // g_group]; beta [B, T, H]; state [N, H, dk, dv].
"""

import numpy as np

__all__ = [
    "expand_decay",
    "kda_step",
    "kda_sequence",
    "kda_forward",
    "kda_decode_step",
]


def expand_decay(g, dk, g_group):
    """Expand grouped log-decay to one value per key channel.

    With g_group == 64 each stored value is shared by 64 consecutive key
    channels (the "decay-g64" ablation of the Mini-K3-1H-decay-g64 card);
    g_group == 1 is KDA's per-channel decay.
    """
    g = np.asarray(g, dtype=np.float64)
    if g.shape[-1] * g_group != dk:
        raise ValueError("g last dim %d * g_group %d != dk %d" % (g.shape[-1], g_group, dk))
    if g_group == 1:
        return g
    return np.repeat(g, g_group, axis=-1)


def kda_step(S, q, k, v, g, beta):
    """One token of the KDA recurrence for a batch of independent heads.

    S: [..., dk, dv] state entering the token; q, k: [..., dk];
    v: [..., dv]; g: [..., dk] (log alpha per key channel, already
    expanded); beta: [...].  Returns (S_t, o_t) as new arrays.

    Steps, in the order of the matrix form:
      1. decay:  S' = Diag(alpha) S             (alpha = exp(g), per key channel)
      2. read:   e  = S'^T k                    (what the decayed state returns for k)
      3. write:  S_t = S' + beta k (v - e)^T    (= (I - beta k k^T) S' + beta k v^T,
                                                 one gradient step on 1/2||S^T k - v||^2)
      4. output: o_t = S_t^T q
    """
    alpha = np.exp(g)
    S_dec = alpha[..., :, None] * S
    e = np.matmul(k[..., None, :], S_dec)[..., 0, :]
    S_new = S_dec + beta[..., None, None] * (k[..., :, None] * (v - e)[..., None, :])
    o = np.matmul(q[..., None, :], S_new)[..., 0, :]
    return S_new, o


def kda_sequence(q, k, v, g, beta, S0):
    """Run the recurrence over a time axis, vectorised over leading heads.

    q, k: [L, ..., dk]; v: [L, ..., dv]; g: [L, ..., dk] (expanded);
    beta: [L, ...]; S0: [..., dk, dv].  Returns (o [L, ..., dv], S_L).
    """
    L = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros(v.shape, dtype=np.float64)
    for t in range(L):
        S, o[t] = kda_step(S, q[t], k[t], v[t], g[t], beta[t])
    return o, S


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kda_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, g_group=1):
    """KDA forward over a batch or a packed (varlen) sequence.

    Without cu_seqlens: B independent sequences of length T; returns
    (o [B, T, H, dv], ht [B, H, dk, dv]).
    With cu_seqlens (int array [N+1], cu[0] = 0, cu[N] = T, non-decreasing):
    B must be 1; document n covers tokens cu[n]..cu[n+1]-1, starts from
    h0[n] (zeros if h0 is None) and its final state is ht[n].
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    g = expand_decay(g, dk, g_group)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    if cu_seqlens is None:
        S0 = np.zeros((B, H, dk, dv)) if h0 is None else _f64(h0)
        # time-major views: [T, B, H, D]
        tm = lambda x: np.moveaxis(x, 1, 0)
        o_tm, ht = kda_sequence(tm(q), tm(k), tm(v), tm(g), tm(beta), S0)
        o[:] = np.moveaxis(o_tm, 0, 1)
        return o, ht
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    N = len(cu) - 1
    ht = np.zeros((N, H, dk, dv)) if h0 is None else np.array(_f64(h0), copy=True)
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        S0 = np.zeros((H, dk, dv)) if h0 is None else _f64(h0[n])
        if b == a:
            ht[n] = S0
            continue
        o_doc, ht[n] = kda_sequence(q[0, a:b], k[0, a:b], v[0, a:b], g[0, a:b], beta[0, a:b], S0)
        o[0, a:b] = o_doc
    return o, ht


def kda_decode_step(state, q, k, v, g, beta, g_group=1):
    """One decode step for N sequences x H heads.

    state: [N, H, dk, dv]; q, k: [N, H, dk]; v: [N, H, dv];
    g: [N, H, dk // g_group]; beta: [N, H].  Returns (new_state, o [N, H, dv]).
    This is the recurrence's single step, the decode form of the
    miniKimiK3 card's KDA bullet (constant cost per token).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    dk = q.shape[-1]
    g = expand_decay(g, dk, g_group)
    return kda_step(_f64(state), q, k, v, g, beta)


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps float32's 8-bit exponent and 8 significant bits (7 stored).
    For a normal value x = m * 2^e with 0.5 <= |m| < 1 (frexp), the nearest
    bfloat16 is round(m * 2^8) * 2^(e - 8) with ties to even, which is what
    numpy's round does.  (Subnormal and overflowing values do not occur in
    the states this is applied to; zeros stay zeros.)
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def round_f16(x):
    """Round float64 values to the nearest IEEE 754 binary16 value, ties to
    even (numpy's float64 -> float16 conversion is that rounding, subnormals
    and overflow to infinity included)."""
    with np.errstate(over="ignore"):  # overflow to infinity is the defined result
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def output_gate(o, z):
    """The output gate on the mixer output: o * sigmoid(z), elementwise.

    The Mini-K3-1H model cards list output gates among the operators the
    family keeps, without a formula; this is the plain reading: an
    elementwise logistic gate with one logit per (sequence, head, value
    channel), the logits z coming from the layer's own gate projection.
    """
    return _f64(o) / (1.0 + np.exp(-_f64(z)))


_STATE_ROUND = {"f32": lambda x: x, "bf16": round_bf16, "f16": round_f16}


def kda_decode_step_pool(pool, slots, q, k, v, g, beta, g_group=1, state_bf16=False, state_dtype=None,
                         o_gate=None):
    """One decode step over a pool of states (serving form).

    pool: [num_slots, H, dk, dv]; slots: [N] ints; q, k: [N, H, dk];
    v: [N, H, dv]; g: [N, H, dk // g_group]; beta: [N, H].
    Sequence n steps the state in pool slot slots[n] (the K3-Tiny-L13 card's
    serving notes: decode concurrency is bounded by a pool of per-sequence
    KDA states whose dtype is a serving knob).  A slot outside [0, num_slots)
    marks the sequence inactive: its output row is zero and no state changes.
    state_dtype "f32" (default), "bf16" (also state_bf16=True) or "f16": the
    pool holds values of that type, the step runs on them exactly and the new
    state is rounded to the nearest value of the type (ties to even).
    o_gate [N, H, dv] or None: the output gate's logits; an active sequence's
    output is then output_gate(o, o_gate).  The output is the exact step's.
    Returns (new_pool, o [N, H, dv]).
    """
    sdt = state_dtype or ("bf16" if state_bf16 else "f32")
    rnd = _STATE_ROUND[sdt]
    pool = _f64(pool).copy()
    slots = np.asarray(slots)
    N, H = np.asarray(q).shape[:2]
    dv = np.asarray(v).shape[-1]
    o = np.zeros((N, H, dv))
    for n in range(N):
        s = int(slots[n])
        if s < 0 or s >= pool.shape[0]:
            continue
        S_new, o_n = kda_decode_step(pool[s][None], np.asarray(q)[n:n + 1], np.asarray(k)[n:n + 1],
                                     np.asarray(v)[n:n + 1], np.asarray(g)[n:n + 1], np.asarray(beta)[n:n + 1],
                                     g_group)
        pool[s] = rnd(S_new[0])
        o[n] = o_n[0] if o_gate is None else output_gate(o_n[0], np.asarray(o_gate)[n])
    return pool, o
