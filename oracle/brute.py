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


def layer(q, k, v, lam, beta, clamp=1e-6, readout=None, gates=None, features_given=False):
    """One (b,h) slice from zero state: q, k [N,F]; v [N,D]; lam, beta [M]; ``readout`` an
    optional complex [M, M] mode-mixing matrix R (a -> a R before the readout; None = identity);
    ``gates`` an optional pair (w, a) of per-token write and decay gates [N] (a > 0): token s
    then enters with weight w_s and is carried to t by prod_{s<u<=t} a_u lambda^(t-s), the
    product taken as exp(sum of log a_u); ``features_given``: q and k are already the features
    phi(q), phi(k) (the layer behind the block's input prologue).

    Returns (o [N,D], num [N,D], den [N]).
    """
    if features_given:
        fq, fk = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    else:
        fq, fk = feature(q), feature(k)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.complex128)
    N = fq.shape[0]
    S = fq @ fk.T                                   # <phi(q_t), phi(k_s)>
    if gates is not None:
        w = np.asarray(gates[0], dtype=np.float64)
        cl = np.cumsum(np.log(np.asarray(gates[1], dtype=np.float64)))   # sum_{u<=t} log a_u
    o = np.empty((N, v.shape[1]))
    num = np.empty_like(o)
    den = np.empty(N)
    for t in range(N):
        dec = powers(lam, t - np.arange(t + 1)) * beta[None, :]     # [s, m] = beta lam^(t-s)
        if gates is not None:
            s = np.arange(t + 1)
            dec = dec * (w[s] * np.exp(cl[t] - cl[s]))[:, None]
        A = (S[t, : t + 1, None] * dec).sum(axis=0)                 # [m]
        Gam = (dec[:, :, None] * v[: t + 1, None, :]).sum(axis=0)   # [m, D]
        eta = dec.sum(axis=0)                                       # [m]
        if readout is not None:
            A = A @ np.asarray(readout, dtype=np.complex128)        # (a R)[n] = sum_m a_m R_mn
        num[t] = np.real((A[:, None] * Gam).sum(axis=0))
        den[t] = np.real((A * eta).sum())
        o[t] = num[t] / max(den[t], clamp)
    return o, num, den


def den_condition(q, k, lam, beta, t, gates=None):
    """The conditioning of the denominator at token t of one slice (from zero state), as
    ``layer`` defines it: den = Re sum_m a_m eta_m, returned with
    kappa = sum_m |Re(a_m eta_m)| / |den|, the factor by which the cancellation in that sum
    amplifies relative errors of its terms (1 when no term cancels another).  A diagnostic for
    tolerances: a recurrence carried in a precision eps resolves den only to about kappa eps.

    Returns (kappa, den)."""
    fq, fk = feature(q), feature(k)
    beta = np.asarray(beta, dtype=np.complex128)
    s = np.arange(t + 1)
    dec = powers(lam, t - s) * beta[None, :]
    if gates is not None:
        w = np.asarray(gates[0], dtype=np.float64)
        cl = np.cumsum(np.log(np.asarray(gates[1], dtype=np.float64)))
        dec = dec * (w[s] * np.exp(cl[t] - cl[s]))[:, None]
    S = fk[: t + 1] @ fq[t]                          # <phi(q_t), phi(k_s)>
    terms = np.real((S[:, None] * dec).sum(axis=0) * dec.sum(axis=0))
    den = terms.sum()
    return float(np.abs(terms).sum() / abs(den)), float(den)


def gated_condition(q, k, v, lam, beta, wgate, dgate, state=None, tokens=None):
    """The conditioning of the readout sums of the gated layer (``layer`` with gates, any real
    gates, zeros and negative values included), at every token t of one slice.  Unrolled, the
    denominator is a sum over triples (s, j, m) -- key s through A, key j through eta, mode m
    -- of phi(q_t).phi(k_s) g_s g_j beta_m^2 lambda_m^(2t-s-j), with g_s = w_s prod_{s<u<=t} a_u
    (products taken directly), plus the terms of the entries of an initial state (U0, G0, E0),
    carried by lambda^(t+1) prod_{u<=t} a_u; the numerator likewise with v_j[d].  Returned per
    token:
        kappa_den = sum |terms of den| / |den|,
        kappa_num = max_d sum |terms of num[d]| / max_d |num[d]|,
    the factors by which the cancellation in those sums amplifies relative errors of their
    terms.  An evaluation that rounds each term's factors to a unit roundoff eps (whatever order
    it sums in) has relative errors up to about (kappa_den + kappa_num) eps; the sum over modes
    alone (``den_condition``) is one of its partial sums.  O(t M (F + D)) per token t:
    ``tokens`` limits the evaluation to those tokens (the others are returned as NaN).

    Returns (kappa_den [N], kappa_num [N])."""
    fq, fk = feature(q), feature(k)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.complex128)
    w = np.asarray(wgate, dtype=np.float64)
    a = np.asarray(dgate, dtype=np.float64)
    N = fq.shape[0]
    if state is not None:
        U0, G0, E0 = (np.asarray(x, dtype=np.complex128) for x in state)
    kd, kn = np.full(N, np.nan), np.full(N, np.nan)
    for t in (range(N) if tokens is None else sorted(set(int(x) for x in tokens))):
        r = np.ones(t + 1)                      # prod_{s<u<=t} a_u
        if t > 0:
            r[:t] = np.cumprod(a[t:0:-1])[::-1]
        g = w[: t + 1] * r
        lp = powers(lam, t - np.arange(t + 1))
        dec = lp * beta[None, :] * g[:, None]                       # [s, m]
        dab = np.abs(lp) * np.abs(beta)[None, :] * np.abs(g)[:, None]
        St = fk[: t + 1] @ fq[t]                                    # phi(q_t).phi(k_s)
        A = (St[:, None] * dec).sum(axis=0)
        Aab = (St[:, None] * dab).sum(axis=0)
        Gam = (dec[:, :, None] * v[: t + 1, None, :]).sum(axis=0)
        Gab = (dab[:, :, None] * np.abs(v[: t + 1, None, :])).sum(axis=0)
        eta, eab = dec.sum(axis=0), dab.sum(axis=0)
        if state is not None:
            p = powers(lam, [t + 1])[0] * (r[0] * a[0])             # lam^(t+1) prod_{u<=t} a_u
            A = A + p * (U0 @ fq[t])
            Aab = Aab + np.abs(p) * (np.abs(U0) @ fq[t])
            Gam = Gam + p[:, None] * G0
            Gab = Gab + np.abs(p)[:, None] * np.abs(G0)
            eta = eta + p * E0
            eab = eab + np.abs(p) * np.abs(E0)
        den = np.real((A * eta).sum())
        num = np.real((A[:, None] * Gam).sum(axis=0))
        kd[t] = (Aab * eab).sum() / abs(den)
        kn[t] = (Aab[:, None] * Gab).sum(axis=0).max() / np.abs(num).max()
    return kd, kn


def layer_batched(q, k, v, lam, beta, clamp=1e-6):
    """[B,N,H,X] layout wrapper around ``layer``."""
    B, N, H, _ = q.shape
    o = np.empty(v.shape)
    for b in range(B):
        for h in range(H):
            o[b, :, h] = layer(q[b, :, h], k[b, :, h], v[b, :, h], lam[h], beta[h], clamp)[0]
    return o
