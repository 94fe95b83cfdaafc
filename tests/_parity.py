"""Helpers for GPU-vs-oracle parity tests.

Tolerances (stated for the method's GPU path and applied to o and final
states): float32 inputs: max-abs <= 1e-4; bfloat16 inputs with float32 state
and accumulation: max-abs <= 2e-2 and relative L2 <= 5e-3, with relative L2 =
||x - x_ref||_2 / ||x_ref||_2 over the whole compared tensor.
"""

import numpy as np
import torch

TOL_F32_MAXABS = 1e-4
TOL_BF16_MAXABS = 2e-2
TOL_BF16_RELL2 = 5e-3


def f64(t):
    """Exact float64 up-cast of a tensor's values (CPU numpy)."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").double().numpy()


def errors(got, ref):
    got, ref = f64(got), f64(ref)
    d = got - ref
    maxabs = float(np.max(np.abs(d))) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
    return maxabs, rel


def assert_close(name, got, ref, dtype):
    got64 = f64(got)
    assert np.all(np.isfinite(got64)), "%s: non-finite values" % name
    maxabs, rel = errors(got64, ref)
    print("PARITY %-40s max-abs %.3e rel-L2 %.3e" % (name, maxabs, rel), flush=True)
    if dtype == torch.float32:
        assert maxabs <= TOL_F32_MAXABS, "%s: max-abs %.3e > %.0e" % (name, maxabs, TOL_F32_MAXABS)
    else:
        assert maxabs <= TOL_BF16_MAXABS and rel <= TOL_BF16_RELL2, (
            "%s: max-abs %.3e (<= %.0e), rel-L2 %.3e (<= %.0e)" % (name, maxabs, TOL_BF16_MAXABS, rel,
                                                                  TOL_BF16_RELL2))
    return maxabs, rel


def to_dev(d):
    out = {}
    for k, v in d.items():
        out[k] = v.cuda() if isinstance(v, torch.Tensor) else v
    return out
