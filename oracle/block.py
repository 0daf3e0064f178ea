"""The IA block's edges around the layer -- TEST INFRASTRUCTURE (numpy, fp64).

Only ``tests/`` (and the oracle's own users listed in ``oracle/__init__.py``) use this module.
It shares no code with the HIP library.

The pages build the IA layer into a model block with pieces at its edges, naming them
without formulas:
- short convolutions on the queries and keys and on the values, which carry much of the
  genomic models' gain (paper summary page §5.3; the ablation setup of §B.1, Table 6);
- rotary position embedding on queries and keys in the language models (summary page
  §A.1), which the §D.1 ablation finds of little effect on IA;
- an RMS normalisation with a learned per-head bias applied to the SSM input
  z_t = [xi(k_t), v_t] (AI Radio episode page, "Implementation Details");
- an output gate (summary page §3.3; Base IA of §B.3 omits it).
The readings written out here (each stated where it is implemented):
- short convolution: causal and depthwise along time, W taps per channel, tap 0 on the
  current token, zeros (or a carried state) before the first token, then SiLU;
- RoPE: feature pairs (2i, 2i+1) of a head rotated by the angle p * base^(-2i/F) at
  position p;
- order on q and k: convolution and SiLU, then RoPE, then the feature map xi = elu + 1;
- RMSNorm with bias: z' = g * z / sqrt(mean(z^2) + eps) + b over the F + Dv entries of z_t,
  g and b per head and entry;
- output gate: o' = o * SiLU(g_t), g_t the caller's gate projection of token t.
"""
from __future__ import annotations

import numpy as np


def silu(x):
    """x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def feature(x):
    """elu(x) + 1."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def short_conv(x, w, state=None):
    """Causal depthwise convolution of one sequence: x [N, C], w [C, W] (w[:, tau] multiplies
    the token tau steps back), state [W-1, C] the W-1 tokens before x (oldest first; None:
    zeros).  Returns y [N, C] (before SiLU) and the W-1 last tokens of state ++ x."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, C = x.shape
    W = w.shape[1]
    prev = np.zeros((W - 1, C)) if state is None else np.asarray(state, dtype=np.float64)
    full = np.concatenate([prev, x], axis=0)          # token n of x is row n + W - 1
    y = np.zeros((N, C))
    for n in range(N):
        for tau in range(W):
            y[n] += w[:, tau] * full[n + W - 1 - tau]
    return y, full[len(full) - (W - 1):].copy() if W > 1 else np.zeros((0, C))


def rope(x, positions, base):
    """Rotate feature pairs (2i, 2i+1) of x [N, F] by positions[n] * base^(-2i/F)."""
    x = np.asarray(x, dtype=np.float64)
    N, F = x.shape
    out = np.empty_like(x)
    for n in range(N):
        for i in range(F // 2):
            th = float(positions[n]) * base ** (-2.0 * i / F)
            c, s = np.cos(th), np.sin(th)
            a, b = x[n, 2 * i], x[n, 2 * i + 1]
            out[n, 2 * i] = a * c - b * s
            out[n, 2 * i + 1] = a * s + b * c
    return out


def rmsnorm_bias(z, g, b, eps):
    """Per row of z [N, E]: g * z / sqrt(mean(z^2) + eps) + b."""
    z = np.asarray(z, dtype=np.float64)
    r = np.sqrt(np.mean(z * z, axis=1, keepdims=True) + eps)
    return np.asarray(g, dtype=np.float64)[None, :] * z / r + np.asarray(b, dtype=np.float64)[None, :]


def prologue_slice(q, k, v, conv=None, state=None, rope_base=0.0, pos0=0, norm=None, eps=1e-6):
    """One (b,h) slice: q, k [N, F], v [N, D] raw projections.  conv: (wq [F, W], wk [F, W],
    wv [D, W]) or None; state: the W-1 raw tokens before q, k, v as one [W-1, 2F+D] array
    (q, k, v channels side by side) or None; norm: (g [F+D], b [F+D]) or None.
    Returns (phi(q'), the normalised [phi(k'), v'] split as fk [N, F] and vo [N, D], and the
    new state [W-1, 2F+D] or None)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    N, F = q.shape
    D = v.shape[1]
    new_state = None
    if conv is not None:
        wq, wk, wv = conv
        raw = np.concatenate([q, k, v], axis=1)
        w = np.concatenate([np.asarray(wq), np.asarray(wk), np.asarray(wv)], axis=0)
        y, new_state = short_conv(raw, w, state)
        y = silu(y)
        q, k, v = y[:, :F], y[:, F:2 * F], y[:, 2 * F:]
    if rope_base > 0:
        pos = pos0 + np.arange(N)
        q = rope(q, pos, rope_base)
        k = rope(k, pos, rope_base)
    fq, fk = feature(q), feature(k)
    if norm is not None:
        z = rmsnorm_bias(np.concatenate([fk, v], axis=1), norm[0], norm[1], eps)
        fk, v = z[:, :F], z[:, F:]
    return fq, fk, v, new_state


def prologue(q, k, v, conv=None, state=None, rope_base=0.0, pos0=0, norm=None, eps=1e-6):
    """``prologue_slice`` over a batch: q, k [B, N, H, F], v [B, N, H, D]; conv per head
    (wq [H, F, W], wk [H, F, W], wv [H, D, W]); state [B, H, W-1, 2F+D]; norm (g [H, F+D],
    b [H, F+D]).  Returns fq, fk, vo in the same layouts and the new state."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, N, H, F = q.shape
    D = v.shape[3]
    fq, fk, vo = np.empty(q.shape), np.empty(k.shape), np.empty(v.shape)
    W = conv[0].shape[2] if conv is not None else 1
    st_out = np.zeros((B, H, max(W - 1, 0), 2 * F + D)) if conv is not None else None
    for b in range(B):
        for h in range(H):
            c = None if conv is None else (conv[0][h], conv[1][h], conv[2][h])
            s = None if (state is None or conv is None) else state[b, h]
            nrm = None if norm is None else (norm[0][h], norm[1][h])
            a, bb, cc, ns = prologue_slice(q[b, :, h], k[b, :, h], v[b, :, h], c, s, rope_base,
                                           pos0, nrm, eps)
            fq[b, :, h], fk[b, :, h], vo[b, :, h] = a, bb, cc
            if st_out is not None:
                st_out[b, h] = ns
    return fq, fk, vo, st_out


def gate(o, g):
    """The output gate: o * SiLU(g), elementwise."""
    return np.asarray(o, dtype=np.float64) * silu(g)
