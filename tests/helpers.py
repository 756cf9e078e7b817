"""Comparison helpers shared by the GPU parity tests."""
import sys

import numpy as np
import torch

# tolerances: max-abs error and (max-abs error / max |reference|), both must hold
TOL_BF16 = (2e-2, 1e-2)
TOL_FP32 = (1e-5, 1e-5)


def note(msg):
    """Name the case before a GPU step, flushed, so a crash report points at it."""
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.double().numpy()
    return np.asarray(t, dtype=np.float64)


def compare(got, ref, tol, what=""):
    """Assert |got - ref| <= tol[0] and max|got - ref| / max|ref| <= tol[1]; return stats."""
    g, r = to_np(got), to_np(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    finite = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), finite), what + ": non-finite pattern differs"
    err = np.abs(g[finite] - r[finite])
    max_abs = float(err.max()) if err.size else 0.0
    scale = float(np.abs(r[finite]).max()) if err.size else 1.0
    rel = max_abs / scale if scale > 0 else max_abs
    gv, rv = g[finite].ravel(), r[finite].ravel()
    cos = float(gv @ rv / (np.linalg.norm(gv) * np.linalg.norm(rv) + 1e-300)) if gv.size else 1.0
    stats = dict(max_abs=max_abs, rel=rel, cos=cos)
    assert max_abs <= tol[0] and rel <= tol[1], "%s: %s exceeds %s" % (what, stats, tol)
    return stats


def round_bf16(a):
    """Round a float64 array to bf16 (nearest even) and back, via torch."""
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
