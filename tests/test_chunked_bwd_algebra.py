"""CPU check of the chunkwise decomposition the chunked backward kernels compute, written out in
numpy (fp64) and compared with the oracle's token-recurrence gradients (``oracle.scan_bwd``).

The decomposition (16-token chunks, powers centred at o = C/2), per chunk with start states U_c,
G_c, e_c and the adjoints S^U, S^G, S^e its last state receives from later tokens:
  a_i  = beta lam^(i-o) (S lam^(o-j))_i + lam^(i+1) phi(q_i) . U_c
  A_i  = beta lam^(i-o) (S' lam^(o-j))_i + lam^(i+1) (g_i . G_c + dd_i e_c),  S' = g V^T + dd 1^T
  P[i,j]  = Re sum_m lam^(i-o) a_i beta lam^(o-j),  Pg likewise with A (both causal)
  dphi(q) = Pg phi(K) + Re(lam^(i+1) A) U_c,  dphi(k) = Pg^T phi(Q) + Re conj(beta lam^(C-1-j)) S^U,
  dv = P^T g + Re conj(beta lam^(C-1-j)) S^G
  S^U <- conj(lam^C) S^U + conj(sum_i lam^(i+1) A_i phi(q_i)), likewise S^G, S^e
with dbeta and dlambda from the per-token adjoints (the distance-weighted sums as
lam^(i-1-o) (i T0 - T1), T0 = S lam^(o-j), T1 = S j lam^(o-j)).  A mistake in any of these
(a dropped carry term, a wrong power, a missing conjugate) fails these cases at 1e-9 or worse.
Sources: "Interdomain Attention: Beyond Token-Level Key-Value Memory", summary page §3.1-§3.2
(recurrence, readout), §A.2 (chunkwise form); episode page, derivation.
"""
import numpy as np
import pytest

import oracle


def _phi(x):
    return np.where(x > 0, x + 1, np.exp(np.minimum(x, 0)))


def chunked_grads(q, k, v, lam, beta, dO, state=None, clamp=1e-6, C=16, no_den=False):
    N, F = q.shape
    D, M, O = v.shape[1], len(lam), C // 2
    nch = (N + C - 1) // C
    pad = nch * C - N
    Q = np.vstack([_phi(q), np.zeros((pad, F))])
    K = np.vstack([_phi(k), np.zeros((pad, F))])
    V = np.vstack([v, np.zeros((pad, D))])
    DO = np.vstack([dO, np.zeros((pad, D))])
    pw = lambda e: lam ** e
    W0 = np.stack([pw(O - j) for j in range(C)])
    W1 = np.stack([j * pw(O - j) for j in range(C)])
    Wt = beta[None] * W0
    Wend = np.stack([beta * pw(C - 1 - j) for j in range(C)])
    W0end = np.stack([pw(C - 1 - j) for j in range(C)])
    E0T = np.stack([sum(pw(e) for e in range(i + 1)) for i in range(C)])
    li = np.stack([pw(i - O) for i in range(C)])
    l1 = np.stack([pw(i + 1) for i in range(C)])
    li0 = np.stack([pw(i) for i in range(C)])
    lq1 = np.stack([pw(i - 1 - O) for i in range(C)])
    mask = np.tril(np.ones((C, C)))
    U = np.zeros((M, F), complex) if state is None else state[0].copy()
    G = np.zeros((M, D), complex) if state is None else state[1].copy()
    e = np.zeros(M, complex) if state is None else state[2].copy()
    # forward sweep: chunk start states, per-token den and dL/do . num
    starts, den, gn = [], np.zeros(nch * C), np.zeros(nch * C)
    for c in range(nch):
        sl = slice(c * C, (c + 1) * C)
        starts.append((U.copy(), G.copy(), e.copy()))
        S = mask * (Q[sl] @ K[sl].T)
        Sd = mask * (DO[sl] @ V[sl].T)
        a = beta * li * (S @ W0) + l1 * (Q[sl] @ U.T)
        X = beta * li * (Sd @ W0) + l1 * (DO[sl] @ G.T)
        ei = l1 * e + beta * E0T
        den[sl] = np.real(a * ei).sum(1)
        gn[sl] = np.real(a * X).sum(1)
        U = lam[:, None] ** C * U + beta[:, None] * (W0end.T @ K[sl])
        G = lam[:, None] ** C * G + beta[:, None] * (W0end.T @ V[sl])
        e = lam ** C * e + beta * E0T[C - 1]
    if no_den:
        inv, dd = np.ones(nch * C), np.zeros(nch * C)
    else:
        inv = 1 / np.maximum(den, clamp)
        dd = np.where(den >= clamp, -gn * inv * inv, 0.0)
    inv[N:] = 0
    dd[N:] = 0
    GG = DO * inv[:, None]
    # reverse sweep
    SU, SG, SE = np.zeros((M, F), complex), np.zeros((M, D), complex), np.zeros(M, complex)
    dq, dk, dv = np.zeros((nch * C, F)), np.zeros((nch * C, F)), np.zeros((nch * C, D))
    dl, db = np.zeros(M, complex), np.zeros(M, complex)
    ii = np.arange(C)[:, None]
    wc = (C - 1 - ii).astype(float)
    wpw = np.stack([beta * pw(C - 2 - j) if j < C - 1 else 0 * beta for j in range(C)])
    for c in reversed(range(nch)):
        sl = slice(c * C, (c + 1) * C)
        Uc, Gc, ec = starts[c]
        ddc = dd[sl]
        S = mask * (Q[sl] @ K[sl].T)
        Sg = mask * (GG[sl] @ V[sl].T + ddc[:, None])
        T0, T1, T0g, T1g = S @ W0, S @ W1, Sg @ W0, Sg @ W1
        T2 = Q[sl] @ Uc.T
        T2g = GG[sl] @ Gc.T + ddc[:, None] * ec[None]
        E, Eg = li * T0, li * T0g
        a = beta * E + l1 * T2
        A = beta * Eg + l1 * T2g
        P = np.real((li * a) @ Wt.T) * mask
        Pg = np.real((li * A) @ Wt.T) * mask
        dq[sl] = Pg @ K[sl] + np.real((l1 * A) @ Uc)
        dk[sl] = Pg.T @ Q[sl] + np.real(np.conj(Wend) @ SU)
        dv[sl] = P.T @ GG[sl] + np.real(np.conj(Wend) @ SG)
        db += np.conj(A * E + a * Eg).sum(0)
        D1, D1g = lq1 * (ii * T0 - T1), lq1 * (ii * T0g - T1g)
        s = beta * (A * D1 + a * D1g) + (ii + 1) * li0 * (A * T2 + a * T2g)
        zz = (SU @ K[sl].T + SG @ V[sl].T + SE[:, None]).T
        db += (zz * np.conj(W0end)).sum(0)
        s = s + wc * np.conj(zz) * wpw
        dot = (SU * np.conj(Uc)).sum(1) + (SG * np.conj(Gc)).sum(1) + SE * np.conj(ec)
        dl += np.conj(s).sum(0) + C * dot * np.conj(lam ** (C - 1))
        SE = np.conj(lam ** C) * SE + np.conj(((l1 * a) * ddc[:, None]).sum(0))
        SU = np.conj(lam[:, None] ** C) * SU + np.conj((l1 * A).T @ Q[sl])
        SG = np.conj(lam[:, None] ** C) * SG + np.conj((l1 * a).T @ GG[sl])
    dphi = lambda x: np.minimum(1.0, _phi(x))
    return dq[:N] * dphi(q), dk[:N] * dphi(k), dv[:N], dl, db, (SU, SG, SE)


@pytest.mark.parametrize("N,F,D,M,with_state,no_den", [
    (37, 8, 8, 4, False, False), (64, 16, 16, 8, True, False), (50, 8, 12, 6, True, True),
    (16, 8, 8, 4, False, False), (5, 8, 8, 4, True, False), (90, 8, 8, 5, False, False)])
def test_chunked_decomposition_matches_the_recurrence(N, F, D, M, with_state, no_den):
    rng = np.random.default_rng(N + 7 * M)
    q, k = rng.normal(size=(N, F)) * 0.5, rng.normal(size=(N, F)) * 0.5
    v, dO = rng.normal(size=(N, D)), rng.normal(size=(N, D))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), M))
    lam = np.exp(dt * (-0.5 + 1j * np.pi * np.arange(M)))
    beta = (rng.normal(size=M) + 1j * rng.normal(size=M)) * 0.3 + 1
    st = None
    if with_state:
        st = (rng.normal(size=(M, F)) * 0.1 + 1j * rng.normal(size=(M, F)) * 0.1 + 0.5,
              rng.normal(size=(M, D)) + 1j * rng.normal(size=(M, D)),
              rng.normal(size=M) * 0.1 + 1 + 0.1j)
    ref = oracle.scan_bwd(q, k, v, lam, beta, dO, state=st, no_den=no_den)
    got = chunked_grads(q, k, v, lam, beta, dO, state=st, no_den=no_den)
    for name, x, r in zip(("dq", "dk", "dv", "dlam", "dbeta"), got[:5], ref[:5]):
        err = np.max(np.abs(x - r)) / np.max(np.abs(r))
        assert err < 1e-9, (name, err)
    for x, r in zip(got[5], ref[5]):   # the initial state's gradient: the adjoints left
        # (without the denominator the eta adjoint is exactly zero on both sides)
        assert np.max(np.abs(x - r)) <= 1e-9 * max(np.max(np.abs(r)), 1e-300)
