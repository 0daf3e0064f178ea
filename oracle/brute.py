"""Brute-force IA layer for tiny inputs -- TEST INFRASTRUCTURE (numpy, fp64).

Evaluates the layer from its unrolled definition rather than from the recurrence: unrolling
the S4D recurrence of the pages (paper summary page §3.2; AI Radio episode page, "Key
Components and Derivation") from a zero state gives, for query position t and mode m,

    A[t, m]     = sum_{s<=t} lambda_m^(t-s) beta_m <phi(q_t), phi(k_s)>
    Gamma_t[m]  = sum_{s<=t} lambda_m^(t-s) beta_m v_s
    eta_t[m]    = sum_{s<=t} lambda_m^(t-s) beta_m
    o_t         = Re(sum_m A[t,m] Gamma_t[m]) / max(Re(sum_m A[t,m] eta_t[m]), clamp)

Powers lambda^n are taken as exp(n Log lambda), never by repeated multiplication, so this
shares no rounding path with the recurrence.  Cost O(N^2 M (F + D)): tiny N only.
"""
from __future__ import annotations

import numpy as np


def feature(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def powers(lam, n):
    """lam^n for every mode and every n in the integer array ``n`` (shape [len(n), M])."""
    lam = np.asarray(lam, dtype=np.complex128)
    return np.exp(np.asarray(n, dtype=np.float64)[:, None] * np.log(lam)[None, :])


def layer(q, k, v, lam, beta, clamp=1e-6, readout=None):
    """One (b,h) slice from zero state: q, k [N,F]; v [N,D]; lam, beta [M]; ``readout`` an
    optional complex [M, M] mode-mixing matrix R (a -> a R before the readout; None = identity).

    Returns (o [N,D], num [N,D], den [N]).
    """
    fq, fk = feature(q), feature(k)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.complex128)
    N = fq.shape[0]
    S = fq @ fk.T                                   # <phi(q_t), phi(k_s)>
    o = np.empty((N, v.shape[1]))
    num = np.empty_like(o)
    den = np.empty(N)
    for t in range(N):
        dec = powers(lam, t - np.arange(t + 1)) * beta[None, :]     # [s, m] = beta lam^(t-s)
        A = (S[t, : t + 1, None] * dec).sum(axis=0)                 # [m]
        Gam = (dec[:, :, None] * v[: t + 1, None, :]).sum(axis=0)   # [m, D]
        eta = dec.sum(axis=0)                                       # [m]
        if readout is not None:
            A = A @ np.asarray(readout, dtype=np.complex128)        # (a R)[n] = sum_m a_m R_mn
        num[t] = np.real((A[:, None] * Gam).sum(axis=0))
        den[t] = np.real((A * eta).sum())
        o[t] = num[t] / max(den[t], clamp)
    return o, num, den


def layer_batched(q, k, v, lam, beta, clamp=1e-6):
    """[B,N,H,X] layout wrapper around ``layer``."""
    B, N, H, _ = q.shape
    o = np.empty(v.shape)
    for b in range(B):
        for h in range(H):
            o[b, :, h] = layer(q[b, :, h], k[b, :, h], v[b, :, h], lam[h], beta[h], clamp)[0]
    return o
