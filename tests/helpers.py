"""Shared helpers of the GPU tests: device transfer and the error metric.

Error metric (the tolerance rule for this layer): row-wise infinity-norm relative error, i.e.
max over rows (b, t, h) of max_j |o - o_ref| / max_j |o_ref|.  Bounds: 2e-3 when the inputs
and the state are fp32, 2e-2 with bf16 inputs.
"""
import numpy as np

TOL_F32 = 2e-3
TOL_BF16 = 2e-2


def dev(x, dtype=None):
    """numpy -> cuda tensor; float arrays become `dtype` (float32 or bfloat16)."""
    import torch
    x = np.asarray(x)
    if np.iscomplexobj(x):
        return torch.from_numpy(np.ascontiguousarray(x.astype(np.complex64))).cuda()
    t = torch.from_numpy(np.ascontiguousarray(x.astype(np.float32)))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    import torch
    if t.is_complex():
        return t.cpu().numpy().astype(np.complex128)
    return t.float().cpu().numpy().astype(np.float64)


def rowrel(o, ref, floor=1e-30):
    """max over rows of max_j |o - ref| / max_j |ref| (rows = all but the last axis)."""
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.max(np.abs(o - ref), axis=-1)
    scale = np.maximum(np.max(np.abs(ref), axis=-1), floor)
    r = err / scale
    if np.any(np.isnan(o) != np.isnan(ref)):
        return np.inf
    return float(np.nanmax(r)) if r.size else 0.0


def state_rel(st, ref):
    """Relative error of each state tensor, normalised per (b,h) slice by its max modulus."""
    out = []
    for a, b in zip(st, ref):
        a = np.asarray(a).reshape(a.shape[0], a.shape[1], -1)
        b = np.asarray(b).reshape(b.shape[0], b.shape[1], -1)
        scale = np.maximum(np.max(np.abs(b), axis=-1), 1e-30)
        out.append(float(np.max(np.max(np.abs(a - b), axis=-1) / scale)))
    return max(out)


def tag(msg):
    """Print a line naming the case, flushed, before a GPU step."""
    print(f"[case] {msg}", flush=True)


def report(name, err):
    """Print a measured error (visible with pytest -s, and in the log on failure)."""
    print(f"[err] {name}: {err:.3e}", flush=True)
