"""CPU oracle for the Interdomain Attention (IA) layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product (``ssm_sequence_mixer_amd``) never does, and this package
never imports the product.  It shares no code with the HIP library.

Two independent implementations live here:

* ``ia_oracle.c`` (loaded through ctypes): the token-by-token fp64 complex recurrence and
  readout, serial, one (b,h) slice per call.  ``prefill``/``decode_step``/``bidir`` below only
  loop over slices and marshal arrays.
* ``brute.py``: the explicit double sum over s <= t and modes m, in numpy, for tiny inputs.

``scan_gated``/``prefill_gated`` run the layer with selective writing and memory decay (a
write gate and a decay gate per token), pinned in ``tests/test_oracle.py``.

``block.py`` (numpy) holds the pieces at the layer's edges in the model block (short
convolutions, RoPE, the RMS normalisation of the SSM input, the output gate), pinned in
``tests/test_oracle_block.py``.

``scan_bwd``/``prefill_bwd`` give the gradients of the same layer (``ia_oracle_scan_bwd``:
reverse-mode differentiation of the recurrence, every forward state kept), pinned to the
forward oracle by finite differences in ``tests/test_oracle_bwd.py``.

The method both follow is stated in the header of ``ia_oracle.c``; the sources are the two
pages titled "Interdomain Attention: Beyond Token-Level Key-Value Memory" (the paper summary
page, sections 3.1-3.2, and the AI Radio episode page, "Key Components and Derivation").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ia_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libia_oracle.so")
_lib = None

GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99", "-fPIC",
           "-shared", "-o", _LIB_PATH, _SRC, "-lm"]


def build() -> None:
    """Compile ia_oracle.c into libia_oracle.so beside it."""
    subprocess.check_call(GCC_CMD)


def load_library(path):
    """ctypes handle of a built ia_oracle.c with its signature declared."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.ia_oracle_scan.restype = ctypes.c_int
    lib.ia_oracle_scan.argtypes = [ctypes.c_int] * 4 + [dp] * 5 + [dp] * 3 + [dp] * 3 + [
        ctypes.c_double]
    lib.ia_oracle_scan_readout.restype = ctypes.c_int
    lib.ia_oracle_scan_readout.argtypes = [ctypes.c_int] * 4 + [dp] * 6 + [dp] * 3 + [dp] * 3 + [
        ctypes.c_double, dp]
    lib.ia_oracle_scan_gated.restype = ctypes.c_int
    lib.ia_oracle_scan_gated.argtypes = [ctypes.c_int] * 4 + [dp] * 7 + [dp] * 3 + [dp] * 3 + [
        ctypes.c_double]
    lib.ia_oracle_scan_bwd.restype = ctypes.c_int
    lib.ia_oracle_scan_bwd.argtypes = [ctypes.c_int] * 4 + [dp] * 5 + [dp] * 3 + [
        dp, ctypes.c_double, ctypes.c_int] + [dp] * 5 + [dp] * 3 + [dp]
    return lib


def _load():
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB_PATH)
                or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = load_library(_LIB_PATH)
    return _lib


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _c2r(z: np.ndarray) -> np.ndarray:
    """complex array -> float64 array with a trailing (re, im) axis."""
    z = np.asarray(z, dtype=np.complex128)
    return np.ascontiguousarray(np.stack([z.real, z.imag], axis=-1))


def _r2c(a: np.ndarray) -> np.ndarray:
    return a[..., 0] + 1j * a[..., 1]


def scan(q, k, v, lam, beta, state=None, clamp=1e-6, lib=None):
    """Recurrence over one (b,h) slice.

    q, k: [N, F]; v: [N, D]; lam, beta: [M] complex; state: (U [M,F], G [M,D], e [M]) complex
    or None for zeros.  Returns (o [N,D], num [N,D], den [N], (U, G, e)).  ``lib``: another
    build of ia_oracle.c to call instead (the tests use it for deliberately broken copies).
    """
    lib = _load() if lib is None else lib
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    N, F = q.shape
    D = v.shape[1]
    M = len(lam)
    if state is None:
        U = np.zeros((M, F, 2))
        G = np.zeros((M, D, 2))
        e = np.zeros((M, 2))
    else:
        U, G, e = (_c2r(x) for x in state)
    o = np.empty((N, D))
    num = np.empty((N, D))
    den = np.empty((N,))
    lib.ia_oracle_scan(N, F, D, M, _ptr(q), _ptr(k), _ptr(v), _ptr(_c2r(lam)),
                       _ptr(_c2r(beta)), _ptr(U), _ptr(G), _ptr(e), _ptr(o), _ptr(num),
                       _ptr(den), float(clamp))
    return o, num, den, (_r2c(U), _r2c(G), _r2c(e))


def prefill(q, k, v, lam, beta, state=None, clamp=1e-6, slices=None, threads=1):
    """Causal IA layer forward over a batch.

    q, k: [B, N, H, F]; v: [B, N, H, D]; lam, beta: [H, M] complex; state: (U [B,H,M,F],
    G [B,H,M,D], e [B,H,M]) complex or None.  ``slices``: optional list of (b, h) to compute
    (others are left NaN).  Returns (o [B,N,H,D], num, den [B,N,H], state).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, F = q.shape
    D = v.shape[3]
    M = lam.shape[1]
    o = np.full((B, N, H, D), np.nan)
    num = np.full((B, N, H, D), np.nan)
    den = np.full((B, N, H), np.nan)
    U = np.full((B, H, M, F), np.nan, dtype=np.complex128)
    G = np.full((B, H, M, D), np.nan, dtype=np.complex128)
    e = np.full((B, H, M), np.nan, dtype=np.complex128)
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        st = None if state is None else (state[0][b, h], state[1][b, h], state[2][b, h])
        r = scan(q[b, :, h], k[b, :, h], v[b, :, h], lam[h], beta[h], st, clamp)
        return bh, r

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(one, todo))
    else:
        results = [one(bh) for bh in todo]
    for (b, h), (ob, nb, db, (Ub, Gb, eb)) in results:
        o[b, :, h] = ob
        num[b, :, h] = nb
        den[b, :, h] = db
        U[b, h], G[b, h], e[b, h] = Ub, Gb, eb
    return o, num, den, (U, G, e)


def decode_step(q_t, k_t, v_t, lam, beta, state, clamp=1e-6):
    """One step for every (b,h): q_t, k_t [B,H,F], v_t [B,H,D]; returns (o_t, state)."""
    o, _, _, st = prefill(np.asarray(q_t)[:, None], np.asarray(k_t)[:, None],
                          np.asarray(v_t)[:, None], lam, beta, state, clamp)
    return o[:, 0], st


def bidir(q, k, v, lam, beta, clamp=1e-6, slices=None, threads=1):
    """Bidirectional layer: IA(x) + flip_t(IA(flip_t x)), both from zero state."""
    fwd = prefill(q, k, v, lam, beta, None, clamp, slices, threads)[0]
    fl = lambda a: np.ascontiguousarray(np.asarray(a)[:, ::-1])
    rev = prefill(fl(q), fl(k), fl(v), lam, beta, None, clamp, slices, threads)[0]
    return fwd + rev[:, ::-1]


def scan_bwd(q, k, v, lam, beta, dO, state=None, clamp=1e-6, no_den=False, lib=None):
    """Gradients of one (b,h) slice by reverse-mode differentiation of the recurrence
    (``ia_oracle_scan_bwd``).  q, k [N,F], v and dO [N,D], lam, beta [M] complex, state as in
    ``scan``.  Complex gradients are dL/dRe + i dL/dIm.  Returns (dq, dk, dv, dlam, dbeta,
    (dU0, dG0, de0))."""
    lib = lib or _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    dO = np.ascontiguousarray(dO, dtype=np.float64)
    N, F = q.shape
    D = v.shape[1]
    M = np.asarray(lam).shape[0]
    st = [None] * 3 if state is None else [_c2r(x) for x in state]
    dq, dk = np.empty((N, F)), np.empty((N, F))
    dv = np.empty((N, D))
    dl, db = np.empty((M, 2)), np.empty((M, 2))
    dU, dG, de = np.empty((M, F, 2)), np.empty((M, D, 2)), np.empty((M, 2))
    work = np.empty((N + 1) * M * (F + D + 1) * 2 + N * M * 2 + N * (D + 1))
    rc = lib.ia_oracle_scan_bwd(N, F, D, M, _ptr(q), _ptr(k), _ptr(v), _ptr(_c2r(lam)),
                                _ptr(_c2r(beta)), _ptr(st[0]), _ptr(st[1]), _ptr(st[2]),
                                _ptr(dO), clamp, int(bool(no_den)), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(dl), _ptr(db), _ptr(dU), _ptr(dG), _ptr(de),
                                _ptr(work))
    if rc != 0:
        raise MemoryError("ia_oracle_scan_bwd")
    return dq, dk, dv, _r2c(dl), _r2c(db), (_r2c(dU), _r2c(dG), _r2c(de))


def prefill_bwd(q, k, v, lam, beta, dO, state=None, clamp=1e-6, no_den=False, slices=None,
                threads=1):
    """Gradients of the causal layer over a batch, slice by slice (``scan_bwd``).

    Shapes as in ``prefill``; dO like o.  Returns (dq, dk, dv, dlam [B,H,M], dbeta [B,H,M],
    (dU0, dG0, de0)): lambda and beta gradients per slice (a layer's are their sum over b);
    slices not in ``slices`` are left NaN."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, N, H, F = q.shape
    D = v.shape[3]
    M = lam.shape[1]
    dq = np.full((B, N, H, F), np.nan)
    dk = np.full((B, N, H, F), np.nan)
    dv = np.full((B, N, H, D), np.nan)
    dl = np.full((B, H, M), np.nan, dtype=np.complex128)
    db = np.full((B, H, M), np.nan, dtype=np.complex128)
    dU = np.full((B, H, M, F), np.nan, dtype=np.complex128)
    dG = np.full((B, H, M, D), np.nan, dtype=np.complex128)
    de = np.full((B, H, M), np.nan, dtype=np.complex128)
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        st = None if state is None else (state[0][b, h], state[1][b, h], state[2][b, h])
        return bh, scan_bwd(q[b, :, h], k[b, :, h], v[b, :, h], lam[h], beta[h], dO[b, :, h],
                            st, clamp, no_den)

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(one, todo))
    else:
        results = [one(bh) for bh in todo]
    for (b, h), (a, bk, c, l, be, (u, g, e)) in results:
        dq[b, :, h], dk[b, :, h], dv[b, :, h] = a, bk, c
        dl[b, h], db[b, h], dU[b, h], dG[b, h], de[b, h] = l, be, u, g, e
    return dq, dk, dv, dl, db, (dU, dG, de)


def bidir_bwd(q, k, v, lam, beta, dO, clamp=1e-6, no_den=False, slices=None, threads=1):
    """Gradients of ``bidir`` (o = IA(x) + flip_t(IA(flip_t x)), both from zero state): the
    causal gradients for dO plus, flipped back, those of the reversed sequence for flip_t(dO).
    Returns (dq, dk, dv, dlam [B,H,M], dbeta [B,H,M])."""
    fl = lambda a: np.ascontiguousarray(np.asarray(a)[:, ::-1])
    f = prefill_bwd(q, k, v, lam, beta, dO, None, clamp, no_den, slices, threads)
    r = prefill_bwd(fl(q), fl(k), fl(v), lam, beta, fl(dO), None, clamp, no_den, slices, threads)
    return (f[0] + r[0][:, ::-1], f[1] + r[1][:, ::-1], f[2] + r[2][:, ::-1], f[3] + r[3],
            f[4] + r[4])


def scan_readout(q, k, v, lam, beta, readout, state=None, clamp=1e-6, lib=None):
    """``scan`` with a complex [M, M] readout matrix R (``ia_oracle_scan_readout``): the
    readouts use a R in place of a.  Returns (o, num, den, (U, G, e))."""
    lib = lib or _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    N, F = q.shape
    D = v.shape[1]
    M = np.asarray(lam).shape[0]
    if state is None:
        U, G, e = np.zeros((M, F, 2)), np.zeros((M, D, 2)), np.zeros((M, 2))
    else:
        U, G, e = (_c2r(x) for x in state)
    o, num, den = np.empty((N, D)), np.empty((N, D)), np.empty(N)
    work = np.empty(4 * M)
    lib.ia_oracle_scan_readout(N, F, D, M, _ptr(q), _ptr(k), _ptr(v), _ptr(_c2r(lam)),
                               _ptr(_c2r(beta)), _ptr(_c2r(readout)), _ptr(U), _ptr(G), _ptr(e),
                               _ptr(o), _ptr(num), _ptr(den), clamp, _ptr(work))
    return o, num, den, (_r2c(U), _r2c(G), _r2c(e))


def prefill_readout(q, k, v, lam, beta, readout, state=None, clamp=1e-6, slices=None,
                    threads=1):
    """``prefill`` with a per-head readout matrix, readout [H, M, M] complex."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, F = q.shape
    D = v.shape[3]
    M = lam.shape[1]
    o = np.full((B, N, H, D), np.nan)
    num = np.full((B, N, H, D), np.nan)
    den = np.full((B, N, H), np.nan)
    U = np.full((B, H, M, F), np.nan, dtype=np.complex128)
    G = np.full((B, H, M, D), np.nan, dtype=np.complex128)
    e = np.full((B, H, M), np.nan, dtype=np.complex128)
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        st = None if state is None else (state[0][b, h], state[1][b, h], state[2][b, h])
        return bh, scan_readout(q[b, :, h], k[b, :, h], v[b, :, h], lam[h], beta[h],
                                readout[h], st, clamp)

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(one, todo))
    else:
        results = [one(bh) for bh in todo]
    for (b, h), (ob, nb, db, (Ub, Gb, eb)) in results:
        o[b, :, h], num[b, :, h], den[b, :, h] = ob, nb, db
        U[b, h], G[b, h], e[b, h] = Ub, Gb, eb
    return o, num, den, (U, G, e)


def scan_gated(q, k, v, lam, beta, wgate, dgate, state=None, clamp=1e-6, lib=None):
    """``scan`` with selective writing and memory decay (``ia_oracle_scan_gated``): per token
    t a write gate wgate[t] on what the token writes and a decay gate dgate[t] on every
    mode's lambda.  Returns (o, num, den, (U, G, e))."""
    lib = lib or _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    wg = np.ascontiguousarray(wgate, dtype=np.float64)
    dg = np.ascontiguousarray(dgate, dtype=np.float64)
    N, F = q.shape
    D = v.shape[1]
    M = np.asarray(lam).shape[0]
    assert wg.shape == (N,) and dg.shape == (N,)
    if state is None:
        U, G, e = np.zeros((M, F, 2)), np.zeros((M, D, 2)), np.zeros((M, 2))
    else:
        U, G, e = (_c2r(x) for x in state)
    o, num, den = np.empty((N, D)), np.empty((N, D)), np.empty(N)
    lib.ia_oracle_scan_gated(N, F, D, M, _ptr(q), _ptr(k), _ptr(v), _ptr(_c2r(lam)),
                             _ptr(_c2r(beta)), _ptr(wg), _ptr(dg), _ptr(U), _ptr(G), _ptr(e),
                             _ptr(o), _ptr(num), _ptr(den), float(clamp))
    return o, num, den, (_r2c(U), _r2c(G), _r2c(e))


def prefill_gated(q, k, v, lam, beta, wgate, dgate, state=None, clamp=1e-6, slices=None,
                  threads=1):
    """``prefill`` with the gates of ``scan_gated``: wgate, dgate [B, N, H]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, F = q.shape
    D = v.shape[3]
    M = lam.shape[1]
    o = np.full((B, N, H, D), np.nan)
    num = np.full((B, N, H, D), np.nan)
    den = np.full((B, N, H), np.nan)
    U = np.full((B, H, M, F), np.nan, dtype=np.complex128)
    G = np.full((B, H, M, D), np.nan, dtype=np.complex128)
    e = np.full((B, H, M), np.nan, dtype=np.complex128)
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        st = None if state is None else (state[0][b, h], state[1][b, h], state[2][b, h])
        return bh, scan_gated(q[b, :, h], k[b, :, h], v[b, :, h], lam[h], beta[h],
                              wgate[b, :, h], dgate[b, :, h], st, clamp)

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(one, todo))
    else:
        results = [one(bh) for bh in todo]
    for (b, h), (ob, nb, db, (Ub, Gb, eb)) in results:
        o[b, :, h], num[b, :, h], den[b, :, h] = ob, nb, db
        U[b, h], G[b, h], e[b, h] = Ub, Gb, eb
    return o, num, den, (U, G, e)
