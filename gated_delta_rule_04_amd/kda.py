"""Python binding of libkda.so (ctypes): argument marshalling only.

Every step of the computation runs in the HIP library; PyTorch provides device
memory and the current HIP stream.  There is no fallback: if the library is
missing or a call fails, an exception is raised.

    o, ht = chunk_fwd(q, k, v, g, beta, initial_state=None, output_final_state=False,
                      cu_seqlens=None)
    o = recurrent_step(q, k, v, g, beta, state)      # state updated in place

Shapes (see include/kda.h): q, k [B, T, H, Dk]; v [B, T, H, Dv];
g [B, T, H, Dk // g_group] (g_group inferred from g's last dim); beta [B, T, H];
states [N, H, Dk, Dv] float32.  Decode: q, k [N, H, Dk]; v [N, H, Dv];
g [N, H, Dk // g_group]; beta [N, H].
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libkda.so")

KDA_F32, KDA_BF16, KDA_F16 = 0, 1, 2
_STATUS = {
    0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
    4: "KDA_ERR_WORKSPACE", 5: "KDA_ERR_UNSUPPORTED", 6: "KDA_ERR_HIP",
}
# KDA_ABI_VERSION of include/kda.h that these bindings are written for.
ABI_VERSION = 10

EXPORTED = ["kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_prologue", "kda_recurrent_step_prologue", "kda_chunk_bwd_workspace_bytes", "kda_chunk_bwd", "kda_chunk_fwd_save", "kda_chunk_bwd_saved", "kda_chunk_bwd_prologue_workspace_bytes", "kda_chunk_bwd_prologue", "kda_recurrent_step", "kda_recurrent_step_pool", "kda_recurrent_step_pool_prologue",
            "kda_short_conv_fwd", "kda_short_conv_bwd_workspace_bytes", "kda_short_conv_bwd", "kda_short_conv_step",
            "kda_status_str", "kda_abi_version"]

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().kda_status_str(status).decode()
        super().__init__("%s failed: %s" % (where, msg))


def lib():
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkda.so not found at %s; build it with "
                           "`python -m gated_delta_rule_04_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.kda_abi_version.restype = i
    L.kda_abi_version.argtypes = []
    L.kda_status_str.restype = ctypes.c_char_p
    L.kda_status_str.argtypes = [i]
    L.kda_chunk_fwd_workspace_bytes.restype = sz
    L.kda_chunk_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    L.kda_chunk_fwd.restype = i
    L.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    L.kda_chunk_fwd_noalloc.restype = i
    L.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    L.kda_chunk_fwd_prologue.restype = i
    L.kda_chunk_fwd_prologue.argtypes = [vp] * 11 + [i, i, i, i, i, i, i, i, vp, sz, vp]
    L.kda_recurrent_step_prologue.restype = i
    L.kda_recurrent_step_prologue.argtypes = [vp] * 9 + [i, i, i, i, i, i, vp]
    L.kda_chunk_bwd_workspace_bytes.restype = sz
    L.kda_chunk_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    L.kda_chunk_bwd.restype = i
    L.kda_chunk_bwd.argtypes = [vp] * 14 + [vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    L.kda_chunk_bwd_saved.restype = i
    L.kda_chunk_bwd_saved.argtypes = [vp] * 14 + [vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    L.kda_chunk_fwd_save.restype = i
    L.kda_chunk_fwd_save.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    L.kda_recurrent_step.restype = i
    L.kda_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    L.kda_recurrent_step_pool.restype = i
    L.kda_recurrent_step_pool.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i, i, i, i, vp]
    L.kda_recurrent_step_pool_prologue.restype = i
    L.kda_recurrent_step_pool_prologue.argtypes = [vp] * 9 + [i, vp, vp, i, i, i, i, i, i, i, vp]
    L.kda_short_conv_fwd.restype = i
    L.kda_short_conv_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    L.kda_chunk_bwd_prologue_workspace_bytes.restype = sz
    L.kda_chunk_bwd_prologue_workspace_bytes.argtypes = [i] * 9
    L.kda_chunk_bwd_prologue.restype = i
    L.kda_chunk_bwd_prologue.argtypes = [vp] * 19 + [i] * 8 + [vp, sz, vp]
    L.kda_short_conv_bwd_workspace_bytes.restype = sz
    L.kda_short_conv_bwd_workspace_bytes.argtypes = [i, i, i, i]
    L.kda_short_conv_bwd.restype = i
    L.kda_short_conv_bwd.argtypes = [vp] * 9 + [i] * 6 + [vp, sz, vp]
    L.kda_short_conv_step.restype = i
    L.kda_short_conv_step.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    _lib = L
    return L


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t, shape, name):
    """Raise ValueError unless tensor t (if given) has exactly this shape.  The
    kernels size every access from q's sizes, so a smaller tensor would be
    read or written out of bounds on the device."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _prefill_shapes(q, k, v, g, beta, g_name="g"):
    """Sizes (B, T, H, Dk, Dv, g_group) of a prefill call, after checking that
    k, v, g and beta agree with q."""
    if q.dim() != 4 or v.dim() != 4 or g.dim() != 4:
        raise ValueError("q, k, v and %s must be 4-d [B, T, H, D]" % g_name)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if g.shape[-1] <= 0 or Dk % g.shape[-1]:
        raise ValueError("%s's last dim must divide Dk" % g_name)
    _expect(k, (B, T, H, Dk), "k")
    _expect(v, (B, T, H, Dv), "v")
    _expect(g, (B, T, H, g.shape[-1]), g_name)
    _expect(beta, (B, T, H), "beta")
    return B, T, H, Dk, Dv, Dk // g.shape[-1]


def _decode_shapes(q, k, v, g, beta, g_name="g"):
    """Sizes (N, H, Dk, Dv, g_group) of a decode call, after checking that
    k, v, g and beta agree with q."""
    if q.dim() != 3 or v.dim() != 3 or g.dim() != 3:
        raise ValueError("q, k, v and %s must be 3-d [N, H, D]" % g_name)
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    if g.shape[-1] <= 0 or Dk % g.shape[-1]:
        raise ValueError("%s's last dim must divide Dk" % g_name)
    _expect(k, (N, H, Dk), "k")
    _expect(v, (N, H, Dv), "v")
    _expect(g, (N, H, g.shape[-1]), g_name)
    _expect(beta, (N, H), "beta")
    return N, H, Dk, Dv, Dk // g.shape[-1]


def _num_seqs(B, cu_seqlens):
    if cu_seqlens is None:
        return B
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise TypeError("cu_seqlens must be a 1-d int32 tensor [num_seqs + 1]")
    if B != 1:
        raise ValueError("packed documents (cu_seqlens) need B == 1")
    return cu_seqlens.numel() - 1


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_bytes(B, T, H, Dk, Dv, num_seqs, varlen, dtype):
    return int(lib().kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, num_seqs, int(bool(varlen)),
                                                   KDA_BF16 if dtype == torch.bfloat16 else KDA_F32))


def chunk_fwd(q, k, v, g, beta, initial_state=None, output_final_state=False, cu_seqlens=None, out=None,
              final_state=None, workspace=None):
    """Chunked KDA prefill.  Returns (o, ht) -- ht is None unless requested."""
    B, T, H, Dk, Dv, g_group = _prefill_shapes(q, k, v, g, beta)
    dt = _dt(q)
    for t in (k, v, g, beta):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, g, beta must share one dtype")
    if initial_state is not None and initial_state.dtype != torch.float32:
        raise TypeError("initial_state must be float32")
    N = _num_seqs(B, cu_seqlens)
    _expect(initial_state, (N, H, Dk, Dv), "initial_state")
    _expect(out, (B, T, H, Dv), "out")
    _expect(final_state, (N, H, Dk, Dv), "final_state")
    if out is not None and out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    if final_state is not None and final_state.dtype != torch.float32:
        raise TypeError("final_state must be float32")
    _check_dev(q, k, v, g, beta, initial_state, cu_seqlens)
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    ht = final_state
    if output_final_state and ht is None:
        ht = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _check_dev(o, ht)
    need = workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, q.dtype)
    ws = workspace
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
                             _ptr(ht), _ptr(cu_seqlens), N, B, T, H, Dk, Dv, g_group, dt, _ptr(ws),
                             0 if ws is None else ws.numel() * ws.element_size(), _stream())
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd")
    return o, ht


def _gate_params(A_log, dt_bias, H, n):
    for t in (A_log, dt_bias):
        if t.dtype != torch.float32 or tuple(t.shape) != (H, n):
            raise TypeError("A_log and dt_bias must be float32 [H, Dk / g_group]")
        if not t.is_contiguous():
            raise ValueError("A_log and dt_bias must be contiguous")


def chunk_fwd_prologue(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, initial_state=None, output_final_state=False,
                       cu_seqlens=None, out=None, final_state=None, workspace=None):
    """Chunked prefill with the fused prologue (bf16): q, k L2-normalised per
    token, g = -exp(A_log) softplus(f + dt_bias), beta = sigmoid(b_raw), all
    inside the kernel.  Returns (o, ht)."""
    B, T, H, Dk, Dv, g_group = _prefill_shapes(q_raw, k_raw, v, f, b_raw, g_name="f")
    dt = _dt(q_raw)
    for t in (k_raw, v, f, b_raw):
        if t.dtype != q_raw.dtype:
            raise TypeError("q_raw, k_raw, v, f, b_raw must share one dtype")
    _gate_params(A_log, dt_bias, H, f.shape[-1])
    if initial_state is not None and initial_state.dtype != torch.float32:
        raise TypeError("initial_state must be float32")
    N = _num_seqs(B, cu_seqlens)
    _expect(initial_state, (N, H, Dk, Dv), "initial_state")
    _expect(out, (B, T, H, Dv), "out")
    _expect(final_state, (N, H, Dk, Dv), "final_state")
    if out is not None and out.dtype != q_raw.dtype:
        raise TypeError("out must have q_raw's dtype")
    if final_state is not None and final_state.dtype != torch.float32:
        raise TypeError("final_state must be float32")
    _check_dev(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, initial_state, cu_seqlens)
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=q_raw.dtype, device=q_raw.device)
    ht = final_state
    if output_final_state and ht is None:
        ht = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q_raw.device)
    _check_dev(o, ht)
    need = workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, q_raw.dtype)
    ws = workspace
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q_raw.device)
    st = lib().kda_chunk_fwd_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(f), _ptr(b_raw), _ptr(A_log),
                                      _ptr(dt_bias), _ptr(initial_state), _ptr(o), _ptr(ht), _ptr(cu_seqlens), N, B,
                                      T, H, Dk, Dv, g_group, dt, _ptr(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(), _stream())
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_prologue")
    return o, ht


def recurrent_step_prologue(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, state, out=None):
    """One decode step with the fused prologue; state [N, H, Dk, Dv] float32
    updated in place.  Returns o [N, H, Dv]."""
    N, H, Dk, Dv, g_group = _decode_shapes(q_raw, k_raw, v, f, b_raw, g_name="f")
    dt = _dt(q_raw)
    for t in (k_raw, v, f, b_raw):
        if t.dtype != q_raw.dtype:
            raise TypeError("q_raw, k_raw, v, f, b_raw must share one dtype")
    _gate_params(A_log, dt_bias, H, f.shape[-1])
    if state.dtype != torch.float32:
        raise TypeError("state must be float32")
    _expect(state, (N, H, Dk, Dv), "state")
    _expect(out, (N, H, Dv), "out")
    if out is not None and out.dtype != q_raw.dtype:
        raise TypeError("out must have q_raw's dtype")
    o = out if out is not None else torch.empty((N, H, Dv), dtype=q_raw.dtype, device=q_raw.device)
    _check_dev(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, state, o)
    st = lib().kda_recurrent_step_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(f), _ptr(b_raw), _ptr(A_log),
                                           _ptr(dt_bias), _ptr(state), _ptr(o), N, H, Dk, Dv, g_group, dt,
                                           _stream())
    if st != 0:
        raise KdaError(st, "kda_recurrent_step_prologue")
    return o


def bwd_workspace_bytes(B, T, H, Dk, Dv, num_seqs, varlen, dtype):
    """Bytes of device workspace chunk_bwd needs."""
    return int(lib().kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, num_seqs, int(bool(varlen)),
                                                   KDA_BF16 if dtype == torch.bfloat16 else KDA_F32))


def chunk_fwd_save(q, k, v, g, beta, initial_state=None, output_final_state=False, cu_seqlens=None, out=None,
                   final_state=None, workspace=None):
    """chunk_fwd (bf16) that also keeps the chunk states for the backward in
    a backward workspace.  Returns (o, ht, workspace); pass the workspace to
    chunk_bwd(..., workspace=..., states_saved=True) with the same inputs."""
    B, T, H, Dk, Dv, g_group = _prefill_shapes(q, k, v, g, beta)
    dt = _dt(q)
    for t in (k, v, g, beta):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, g, beta must share one dtype")
    if initial_state is not None and initial_state.dtype != torch.float32:
        raise TypeError("initial_state must be float32")
    N = _num_seqs(B, cu_seqlens)
    _expect(initial_state, (N, H, Dk, Dv), "initial_state")
    _expect(out, (B, T, H, Dv), "out")
    _expect(final_state, (N, H, Dk, Dv), "final_state")
    if out is not None and out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    if final_state is not None and final_state.dtype != torch.float32:
        raise TypeError("final_state must be float32")
    _check_dev(q, k, v, g, beta, initial_state, cu_seqlens)
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    ht = final_state
    if output_final_state and ht is None:
        ht = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _check_dev(o, ht)
    need = bwd_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, q.dtype)
    ws = workspace
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().kda_chunk_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
                                  _ptr(ht), _ptr(cu_seqlens), N, B, T, H, Dk, Dv, g_group, dt, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream())
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_save")
    return o, ht, ws


def chunk_bwd(q, k, v, g, beta, do, initial_state=None, dht=None, cu_seqlens=None, workspace=None, out=None,
              states_saved=False):
    """Gradients of <do, o> + <dht, ht> for chunk_fwd(q, k, v, g, beta,
    initial_state, cu_seqlens) (bf16 inputs).  Returns a dict with dq, dk,
    dv, dg, dbeta (bf16, shaped like the inputs) and dh0 (float32
    [N, H, Dk, Dv]).  `out` may hold preallocated tensors under those names."""
    B, T, H, Dk, Dv, g_group = _prefill_shapes(q, k, v, g, beta)
    dt = _dt(q)
    for t in (k, v, g, beta, do):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, g, beta, do must share one dtype")
    for t in (initial_state, dht):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("initial_state and dht must be float32")
    N = _num_seqs(B, cu_seqlens)
    _expect(do, (B, T, H, Dv), "do")
    _expect(initial_state, (N, H, Dk, Dv), "initial_state")
    _expect(dht, (N, H, Dk, Dv), "dht")
    out = dict(out or {})
    for name, like in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta)):
        t = out.get(name)
        _expect(t, like.shape, name)
        if t is not None and t.dtype != q.dtype:
            raise TypeError("%s must have q's dtype" % name)
    _expect(out.get("dh0"), (N, H, Dk, Dv), "dh0")
    if out.get("dh0") is not None and out["dh0"].dtype != torch.float32:
        raise TypeError("dh0 must be float32")
    _check_dev(q, k, v, g, beta, do, initial_state, dht, cu_seqlens)
    for name, like in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta)):
        if out.get(name) is None:
            out[name] = torch.empty_like(like)
    if out.get("dh0") is None:
        out["dh0"] = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _check_dev(*out.values())
    need = bwd_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, q.dtype)
    ws = workspace
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if states_saved and workspace is None:
        raise ValueError("states_saved needs the workspace that chunk_fwd_save filled")
    fn = lib().kda_chunk_bwd_saved if states_saved else lib().kda_chunk_bwd
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(do), _ptr(dht),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]),
            _ptr(cu_seqlens), N, B, T, H, Dk, Dv, g_group, dt, _ptr(ws), ws.numel() * ws.element_size(), _stream())
    if st != 0:
        raise KdaError(st, "kda_chunk_bwd_saved" if states_saved else "kda_chunk_bwd")
    return out


def chunk_bwd_prologue(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, do, initial_state=None, dht=None, cu_seqlens=None,
                       workspace=None, out=None):
    """Gradients of <do, o> + <dht, ht> for chunk_fwd_prologue (bf16).
    Returns a dict with dq_raw, dk_raw, dv, df, db_raw (bf16, shaped like
    the inputs), dA_log, ddt_bias (float32 [H, Dk/g_group]) and dh0 (float32
    [N, H, Dk, Dv]).  `out` may hold preallocated tensors under those names."""
    B, T, H, Dk, Dv, g_group = _prefill_shapes(q_raw, k_raw, v, f, b_raw, g_name="f")
    dt = _dt(q_raw)
    for t in (k_raw, v, f, b_raw, do):
        if t.dtype != q_raw.dtype:
            raise TypeError("q_raw, k_raw, v, f, b_raw, do must share one dtype")
    _gate_params(A_log, dt_bias, H, f.shape[-1])
    for t in (initial_state, dht):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("initial_state and dht must be float32")
    N = _num_seqs(B, cu_seqlens)
    _expect(do, (B, T, H, Dv), "do")
    _expect(initial_state, (N, H, Dk, Dv), "initial_state")
    _expect(dht, (N, H, Dk, Dv), "dht")
    like = {"dq_raw": q_raw, "dk_raw": k_raw, "dv": v, "df": f, "db_raw": b_raw, "dA_log": A_log, "ddt_bias": dt_bias}
    given = dict(out or {})
    for name, t in given.items():
        if name not in like and name != "dh0":
            raise ValueError("unknown gradient name %r" % name)
        ref_shape = (N, H, Dk, Dv) if name == "dh0" else tuple(like[name].shape)
        ref_dtype = torch.float32 if name == "dh0" else like[name].dtype
        _expect(t, ref_shape, name)
        if t.dtype != ref_dtype:
            raise TypeError("%s must be %s" % (name, ref_dtype))
    _check_dev(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, do, initial_state, dht, cu_seqlens, *given.values())
    out = {n: given[n] if n in given else torch.empty_like(t) for n, t in like.items()}
    out["dh0"] = given["dh0"] if "dh0" in given else torch.empty((N, H, Dk, Dv), dtype=torch.float32,
                                                                  device=q_raw.device)
    need = int(lib().kda_chunk_bwd_prologue_workspace_bytes(B, T, H, Dk, Dv, N, int(cu_seqlens is not None), g_group,
                                                            dt))
    ws = workspace
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q_raw.device)
    st = lib().kda_chunk_bwd_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(f), _ptr(b_raw), _ptr(A_log),
                                      _ptr(dt_bias), _ptr(initial_state), _ptr(do), _ptr(dht), _ptr(out["dq_raw"]),
                                      _ptr(out["dk_raw"]), _ptr(out["dv"]), _ptr(out["df"]), _ptr(out["db_raw"]),
                                      _ptr(out["dA_log"]), _ptr(out["ddt_bias"]), _ptr(out["dh0"]), _ptr(cu_seqlens),
                                      N, B, T, H, Dk, Dv, g_group, dt, _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream())
    if st != 0:
        raise KdaError(st, "kda_chunk_bwd_prologue")
    return out


def recurrent_step(q, k, v, g, beta, state, out=None):
    """One KDA decode step; `state` [N, H, Dk, Dv] float32 is updated in place."""
    N, H, Dk, Dv, g_group = _decode_shapes(q, k, v, g, beta)
    dt = _dt(q)
    for t in (k, v, g, beta):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, g, beta must share one dtype")
    if state.dtype != torch.float32:
        raise TypeError("state must be float32")
    _expect(state, (N, H, Dk, Dv), "state")
    _expect(out, (N, H, Dv), "out")
    if out is not None and out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    _check_dev(q, k, v, g, beta, state)
    o = out if out is not None else torch.empty((N, H, Dv), dtype=q.dtype, device=q.device)
    st = lib().kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o), N, H, Dk,
                                  Dv, g_group, dt, _stream())
    if st != 0:
        raise KdaError(st, "kda_recurrent_step")
    return o


def recurrent_step_pool(q, k, v, g, beta, state_pool, slots, out=None, o_gate=None):
    """One KDA decode step over a state pool: sequence n updates
    state_pool[slots[n]] in place ([num_slots, H, Dk, Dv], float32, bfloat16
    or float16).  A slot outside [0, num_slots) marks the sequence inactive:
    its output row is zero and no state is touched.  o_gate [N, H, Dv] (q's
    dtype): logits z of the output gate, o <- o * sigmoid(z)."""
    N, H, Dk, Dv, g_group = _decode_shapes(q, k, v, g, beta)
    dt = _dt(q)
    for t in (k, v, g, beta):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, g, beta must share one dtype")
    _expect(out, (N, H, Dv), "out")
    if out is not None and out.dtype != q.dtype:
        raise TypeError("out must have q's dtype")
    sdt = KDA_F16 if state_pool.dtype == torch.float16 else _dt(state_pool)
    if slots.dtype != torch.int32 or slots.shape != (N,):
        raise TypeError("slots must be int32 of shape [N]")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, Dk, Dv):
        raise ValueError("state_pool must be [num_slots, H, Dk, Dv]")
    if o_gate is not None and (o_gate.dtype != q.dtype or tuple(o_gate.shape) != (N, H, Dv)
                               or not o_gate.is_contiguous()):
        raise ValueError("o_gate must be a contiguous [N, H, Dv] tensor of q's dtype")
    _check_dev(q, k, v, g, beta, state_pool, slots, o_gate)
    o = out if out is not None else torch.empty((N, H, Dv), dtype=q.dtype, device=q.device)
    st = lib().kda_recurrent_step_pool(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                       _ptr(slots), state_pool.shape[0], _ptr(o), _ptr(o_gate), N, H, Dk, Dv,
                                       g_group, dt, sdt, _stream())
    if st != 0:
        raise KdaError(st, "kda_recurrent_step_pool")
    return o


def recurrent_step_pool_prologue(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, state_pool, slots, out=None,
                                 o_gate=None):
    """recurrent_step_pool on raw projections: the fused prologue (q, k L2
    norm; g = -exp(A_log) softplus(f + dt_bias); beta = sigmoid(b_raw)) and
    one decode step over a state pool, with the optional output gate."""
    N, H, Dk, Dv, g_group = _decode_shapes(q_raw, k_raw, v, f, b_raw, g_name="f")
    dt = _dt(q_raw)
    for t in (k_raw, v, f, b_raw):
        if t.dtype != q_raw.dtype:
            raise TypeError("q_raw, k_raw, v, f, b_raw must share one dtype")
    _gate_params(A_log, dt_bias, H, f.shape[-1])
    _expect(out, (N, H, Dv), "out")
    if out is not None and out.dtype != q_raw.dtype:
        raise TypeError("out must have q_raw's dtype")
    sdt = KDA_F16 if state_pool.dtype == torch.float16 else _dt(state_pool)
    if slots.dtype != torch.int32 or slots.shape != (N,):
        raise TypeError("slots must be int32 of shape [N]")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, Dk, Dv):
        raise ValueError("state_pool must be [num_slots, H, Dk, Dv]")
    if o_gate is not None and (o_gate.dtype != q_raw.dtype or tuple(o_gate.shape) != (N, H, Dv)):
        raise ValueError("o_gate must be an [N, H, Dv] tensor of q_raw's dtype")
    o = out if out is not None else torch.empty((N, H, Dv), dtype=q_raw.dtype, device=q_raw.device)
    _check_dev(q_raw, k_raw, v, f, b_raw, A_log, dt_bias, state_pool, slots, o, o_gate)
    st = lib().kda_recurrent_step_pool_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(f), _ptr(b_raw),
                                                _ptr(A_log), _ptr(dt_bias), _ptr(state_pool), _ptr(slots),
                                                state_pool.shape[0], _ptr(o), _ptr(o_gate), N, H, Dk, Dv, g_group,
                                                dt, sdt, _stream())
    if st != 0:
        raise KdaError(st, "kda_recurrent_step_pool_prologue")
    return o


def short_conv_fwd(x, weight, conv0=None, output_final_state=False, cu_seqlens=None, out=None, conv_final=None):
    """Short causal depthwise convolution along tokens with document reset.
    x [B, T, C]; weight [C, W]; conv0 / conv_final [N, W-1, C] (same dtype).
    Returns (y, conv_final) -- conv_final is None unless requested."""
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be [B, T, C] and weight [C, W]")
    B, T, C = x.shape
    W = weight.shape[-1]
    dt = _dt(x)
    for t in (weight, conv0, conv_final, out):
        if t is not None and t.dtype != x.dtype:
            raise TypeError("x, weight, conv states and y must share one dtype")
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError("weight must be [C, W]")
    N = _num_seqs(B, cu_seqlens)
    _expect(conv0, (N, max(W - 1, 0), C), "conv0")
    _expect(conv_final, (N, max(W - 1, 0), C), "conv_final")
    _expect(out, (B, T, C), "out")
    y = out if out is not None else torch.empty_like(x)
    cf = conv_final
    if output_final_state and cf is None:
        cf = torch.empty((N, max(W - 1, 0), C), dtype=x.dtype, device=x.device)
    _check_dev(x, weight, conv0, y, cf, cu_seqlens)
    st = lib().kda_short_conv_fwd(_ptr(x), _ptr(weight), _ptr(conv0), _ptr(y), _ptr(cf), _ptr(cu_seqlens), N, B, T,
                                  C, W, dt, _stream())
    if st != 0:
        raise KdaError(st, "kda_short_conv_fwd")
    return y, cf


def short_conv_bwd(x, weight, dy, conv0=None, dconv_final=None, cu_seqlens=None, workspace=None):
    """Gradients of <dy, y> + <dconv_final, conv_final> for short_conv_fwd(x,
    weight, conv0, cu_seqlens).  Returns a dict with dx (x's dtype), dweight
    (float32 [C, W]) and dconv0 (x's dtype [N, W-1, C])."""
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be [B, T, C] and weight [C, W]")
    B, T, C = x.shape
    W = weight.shape[-1]
    dt = _dt(x)
    for t in (weight, conv0, dy, dconv_final):
        if t is not None and t.dtype != x.dtype:
            raise TypeError("x, weight, dy and conv states must share one dtype")
    _expect(weight, (C, W), "weight")
    N = _num_seqs(B, cu_seqlens)
    _expect(dy, (B, T, C), "dy")
    _expect(conv0, (N, max(W - 1, 0), C), "conv0")
    _expect(dconv_final, (N, max(W - 1, 0), C), "dconv_final")
    _check_dev(x, weight, dy, conv0, dconv_final, cu_seqlens)
    out = {"dx": torch.empty_like(x), "dweight": torch.empty((C, W), dtype=torch.float32, device=x.device),
           "dconv0": torch.empty((N, max(W - 1, 0), C), dtype=x.dtype, device=x.device)}
    need = int(lib().kda_short_conv_bwd_workspace_bytes(B, T, C, W))
    ws = workspace
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib().kda_short_conv_bwd(_ptr(x), _ptr(weight), _ptr(conv0), _ptr(dy), _ptr(dconv_final), _ptr(out["dx"]),
                                  _ptr(out["dweight"]), _ptr(out["dconv0"]) if W > 1 and N > 0 else None,
                                  _ptr(cu_seqlens), N, B, T, C, W, dt, _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream())
    if st != 0:
        raise KdaError(st, "kda_short_conv_bwd")
    return out


def short_conv_step(x, weight, conv_state, out=None):
    """One decode step of the short convolution: x [N, C]; conv_state
    [N, W-1, C] updated in place.  Returns y [N, C]."""
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError("x must be [N, C] and weight [C, W]")
    N, C = x.shape
    W = weight.shape[-1]
    dt = _dt(x)
    for t in (weight, conv_state, out):
        if t is not None and t.dtype != x.dtype:
            raise TypeError("x, weight, conv_state and y must share one dtype")
    _expect(weight, (C, W), "weight")
    _expect(conv_state, (N, max(W - 1, 0), C), "conv_state")
    _expect(out, (N, C), "out")
    y = out if out is not None else torch.empty_like(x)
    _check_dev(x, weight, conv_state, y)
    st = lib().kda_short_conv_step(_ptr(x), _ptr(weight), _ptr(conv_state), _ptr(y), N, C, W, dt, _stream())
    if st != 0:
        raise KdaError(st, "kda_short_conv_step")
    return y
