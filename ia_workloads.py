"""Seeded synthetic inputs for the IA layer (shared by the tests, the benchmark and the smoke
check).  This module only draws numbers: it holds none of the layer's arithmetic, and it
imports neither the HIP binding nor the CPU oracle.

Every array is produced on the host with ``numpy.random.default_rng``; q, k, v are drawn in
float32 and rounded to bf16 (round to nearest even) when the workload is bf16, so the values
the GPU receives and the values the oracle receives are the same numbers.

Mode parameters follow the S4D-Lin rule named for the workloads: lambda_{h,m} =
exp(dt_h (-1/2 + i pi m)), m = 0..M-1, with dt_h log-uniform in [1e-3, 1e-1] per head (or a
fixed dt), built in float64 and rounded once to complex64; beta_m = 1.

Workloads (sizes as named for the layer shapes; "d" is the head dim, F = Dv = d):
  tiny       B=1  H=1  N=256     F=Dv=M=16  fp32, q,k,v ~ N(0,1), dt = 0.01
  125m       B=8  H=12 N=2048    F=Dv=M=64  bf16, N(0,1/d)
  1.3b       B=4  H=16 N=2048    F=Dv=128 M=64  bf16, N(0,1/d)
  1.3b_long  as 1.3b with N=7168 (3.5x length), same lambda, new q,k,v
  caduceus   B=2  H=8  N=131072  F=Dv=M=32  bidirectional; one-hot DNA tokens times
             N(0, 0.02^2) projections (4 x 256, split into 8 heads of 32)
  decode     H=16 F=Dv=128 M=64, batch 1/16/64: a 32-token prefill, then 256 steps
"""
from __future__ import annotations

import numpy as np

DT_RANGE = (1e-3, 1e-1)


def round_bf16(x) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def s4d_lin(dt, M) -> np.ndarray:
    """[H, M] complex64 modes exp(dt_h (-1/2 + i pi m))."""
    dt = np.atleast_1d(np.asarray(dt, dtype=np.float64))
    m = np.arange(M, dtype=np.float64)
    lam = np.exp(dt[:, None] * (-0.5 + 1j * np.pi * m[None, :]))
    return lam.astype(np.complex64)


def draw_dt(rng, H, lo=DT_RANGE[0], hi=DT_RANGE[1]) -> np.ndarray:
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=H))


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return round_bf16(x) if dtype == "bf16" else x.astype(np.float32)


def make_inputs(B, H, N, F, D, M, dtype="bf16", seed=0, dt=None, std=None, dt_seed=None,
                beta=None):
    """Generic seeded layer inputs: q, k [B,N,H,F], v [B,N,H,D] (float32 arrays holding
    dtype-exact values), lam, beta [H,M] complex64.

    dt: None = log-uniform per head (drawn first from ``dt_seed`` or ``seed``), a float for
    a fixed dt, or an array of H values.  std: None = 1/sqrt(F).
    """
    rng = np.random.default_rng(seed)
    if dt is None:
        dt_rng = rng if dt_seed is None else np.random.default_rng(dt_seed)
        dt = draw_dt(dt_rng, H)
    dt = np.broadcast_to(np.asarray(dt, dtype=np.float64), (H,))
    std = 1.0 / np.sqrt(F) if std is None else std
    q = _normal(rng, (B, N, H, F), std, dtype)
    k = _normal(rng, (B, N, H, F), std, dtype)
    v = _normal(rng, (B, N, H, D), std, dtype)
    lam = s4d_lin(dt, M)
    b = np.ones((H, M), np.complex64) if beta is None else np.asarray(beta, np.complex64)
    return dict(q=q, k=k, v=v, lam=lam, beta=b, dtype=dtype, dt=dt,
                shape=dict(B=B, H=H, N=N, F=F, D=D, M=M))


def tiny():
    return make_inputs(1, 1, 256, 16, 16, 16, dtype="f32", seed=1, dt=0.01, std=1.0)


def l125m():
    return make_inputs(8, 12, 2048, 64, 64, 64, dtype="bf16", seed=2)


def l1p3b(N=2048):
    if N == 2048:
        return make_inputs(4, 16, 2048, 128, 128, 64, dtype="bf16", seed=3)
    # length-extrapolation run: lambda from the 1.3b draw (seed 3), fresh q, k, v
    return make_inputs(4, 16, N, 128, 128, 64, dtype="bf16", seed=33, dt_seed=3)


def dt_1p3b(H=16):
    return draw_dt(np.random.default_rng(3), H)


def caduceus(B=2, N=131072, H=8, d=32, M=32, seed=4):
    """One-hot DNA tokens over {A,C,G,T} times random N(0, 0.02^2) projections."""
    rng = np.random.default_rng(seed)
    dt = draw_dt(rng, H)
    tokens = rng.integers(0, 4, size=(B, N))
    W = [rng.standard_normal((4, H * d)).astype(np.float32) * np.float32(0.02)
         for _ in range(3)]
    q, k, v = (round_bf16(w[tokens].reshape(B, N, H, d)) for w in W)
    lam = s4d_lin(dt, M)
    return dict(q=q, k=k, v=v, lam=lam, beta=np.ones((H, M), np.complex64), dtype="bf16",
                dt=dt, tokens=tokens, shape=dict(B=B, H=H, N=N, F=d, D=d, M=M))


def decode(B, steps=256, prefix=32, H=16, F=128, D=128, M=64, seed=5):
    """Prefix tokens [B,prefix,H,*] and per-step tokens [steps,B,H,*], bf16 N(0,1/d)."""
    rng = np.random.default_rng([seed, B])
    std = 1.0 / np.sqrt(F)
    pre = {n: _normal(rng, (B, prefix, H, F if n != "v" else D), std, "bf16")
           for n in ("q", "k", "v")}
    stp = {n: _normal(rng, (steps, B, H, F if n != "v" else D), std, "bf16")
           for n in ("q", "k", "v")}
    lam = s4d_lin(dt_1p3b(H), M)
    return dict(prefix=pre, steps=stp, lam=lam, beta=np.ones((H, M), np.complex64),
                dtype="bf16", shape=dict(B=B, H=H, F=F, D=D, M=M, prefix=prefix,
                                         steps=steps))
