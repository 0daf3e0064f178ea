"""GPU parity of the token-by-token kernels (decode step, fp32 prefill) against the oracle.

All inputs are seeded (ia_workloads); the oracle receives the very values the GPU receives.
"""
import numpy as np
import pytest

import ia_workloads as W
import oracle
from helpers import TOL_BF16, TOL_F32, dev, host, report, rowrel, state_rel, tag

pytestmark = pytest.mark.gpu


def _lib():
    import ssm_sequence_mixer_amd as ia
    return ia


def _torch():
    import torch
    return torch


def _oracle_state(B, H, F, D, M, lam, beta, seed):
    """A non-trivial state: the oracle's state after 9 random tokens."""
    inp = W.make_inputs(B, H, 9, F, D, M, dtype="f32", seed=seed, std=0.5)
    _, _, _, st = oracle.prefill(inp["q"], inp["k"], inp["v"], lam, beta)
    return st


@pytest.mark.parametrize("in_dtype,out_dtype", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_decode_steps_match_oracle(in_dtype, out_dtype):
    torch = _torch()
    ia = _lib()
    B, H, F, D, M, steps = 2, 3, 32, 48, 16, 5
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    inp = W.make_inputs(B, H, steps, F, D, M, dtype=in_dtype, seed=11)
    lam, beta = inp["lam"], inp["beta"] * np.complex64(0.7 - 0.2j)
    st_ref = _oracle_state(B, H, F, D, M, lam, beta, seed=12)
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)  # both sides continue from the complex64 state
    for t in range(steps):
        tag(f"decode step {t} {in_dtype}->{out_dtype}")
        o = ia.decode(dev(inp["q"][:, t], tdt[in_dtype]), dev(inp["k"][:, t], tdt[in_dtype]),
                      dev(inp["v"][:, t], tdt[in_dtype]), dev(lam), dev(beta), st,
                      out_dtype=tdt[out_dtype])
        o_ref, st_ref = oracle.decode_step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], lam,
                                           beta, st_ref)
        torch.cuda.synchronize()
        tol = TOL_F32 if out_dtype == "f32" else TOL_BF16
        assert rowrel(host(o), o_ref) < tol
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("shape", [(32, 32, 16), (32, 128, 64), (64, 64, 128), (128, 32, 16),
                                   (64, 128, 32), (128, 128, 64), (128, 128, 128)])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_decode_row_kernel_shapes(shape, in_dtype):
    """Decode at the row widths the row-parallel kernel takes (F, Dv in {32, 64, 128}),
    including passes that cover more rows than there are modes (F=32, M=16)."""
    torch = _torch()
    ia = _lib()
    F, D, M = shape
    B, H, steps = 3, 2, 3
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    inp = W.make_inputs(B, H, steps, F, D, M, dtype=in_dtype, seed=F + D + M)
    lam, beta = inp["lam"], inp["beta"]
    st_ref = _oracle_state(B, H, F, D, M, lam, beta, seed=M + 1)
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    for t in range(steps):
        tag(f"decode rows F={F} D={D} M={M} {in_dtype} step {t}")
        o = ia.decode(dev(inp["q"][:, t], tdt[in_dtype]), dev(inp["k"][:, t], tdt[in_dtype]),
                      dev(inp["v"][:, t], tdt[in_dtype]), dev(lam), dev(beta), st)
        o_ref, st_ref = oracle.decode_step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], lam,
                                           beta, st_ref)
        torch.cuda.synchronize()
        assert rowrel(host(o), o_ref) < TOL_F32
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


def test_fp32_prefill_tiny_workload():
    """The tiny fp32 workload: B=H=1, N=256, F=Dv=M=16, dt=0.01, beta=1; outputs and state."""
    torch = _torch()
    ia = _lib()
    inp = W.tiny()
    tag("fp32 prefill tiny")
    st = ia.new_state(1, 1, 16, 16, 16)
    o = ia.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["lam"]),
                   dev(inp["beta"]), state=st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, _, den_ref, st_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"],
                                               inp["beta"])
    assert np.all(den_ref > 10 * 1e-6)
    assert rowrel(host(o), o_ref) < TOL_F32
    assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("N", [1, 63, 130])
def test_fp32_prefill_ragged_and_resume(N):
    torch = _torch()
    ia = _lib()
    B, H, F, D, M = 2, 2, 32, 16, 32
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=20 + N)
    q, k, v = (dev(inp[n]) for n in "qkv")
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    tag(f"fp32 prefill N={N}")
    st = ia.new_state(B, H, M, F, D)
    o = ia.prefill(q, k, v, lam, beta, state=st, out_dtype=torch.float32)
    o_ref, _, _, st_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])
    torch.cuda.synchronize()
    assert rowrel(host(o), o_ref) < TOL_F32
    assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32
    # state-only prefill of a prefix, then the rest from that state, equals the whole
    if N > 1:
        s = N // 2
        st2 = ia.new_state(B, H, M, F, D)
        ia.prefill(q[:, :s].contiguous(), k[:, :s].contiguous(), v[:, :s].contiguous(), lam,
                   beta, state=st2, want_output=False)
        o2 = ia.prefill(q[:, s:].contiguous(), k[:, s:].contiguous(), v[:, s:].contiguous(),
                        lam, beta, state=st2, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert rowrel(host(o2), o_ref[:, s:]) < TOL_F32
        assert state_rel(tuple(host(x) for x in st2), st_ref) < TOL_F32


def test_fp32_bidirectional():
    torch = _torch()
    ia = _lib()
    B, H, N, F, D, M = 1, 2, 45, 16, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=31)
    tag("fp32 bidir")
    o = ia.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["lam"]),
                   dev(inp["beta"]), bidir=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref = oracle.bidir(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])
    assert rowrel(host(o), o_ref) < TOL_F32


def test_decode_forced_clamp():
    """beta = i with real lambda drives Re(den) below zero: o_t = num / clamp."""
    torch = _torch()
    ia = _lib()
    B, H, F, D, M = 1, 1, 16, 16, 16
    lam = np.full((H, M), 0.9, np.complex64)
    beta = np.full((H, M), 1j, np.complex64)
    inp = W.make_inputs(B, H, 3, F, D, M, dtype="f32", seed=41)
    st = ia.new_state(B, H, M, F, D)
    st_ref = tuple(np.zeros(s, np.complex128) for s in ((B, H, M, F), (B, H, M, D), (B, H, M)))
    for t in range(3):
        tag(f"decode clamp step {t}")
        o = ia.decode(dev(inp["q"][:, t]), dev(inp["k"][:, t]), dev(inp["v"][:, t]), dev(lam),
                      dev(beta), st)
        o_ref, st_ref = oracle.decode_step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], lam,
                                           beta, st_ref)
        torch.cuda.synchronize()
        assert np.all(np.abs(o_ref) > 1e3)  # the clamp was hit
        assert rowrel(host(o), o_ref) < TOL_F32


@pytest.mark.parametrize("Bd", [1, 16, 64])
def test_decode_1p3b_shape(Bd):
    """Decode at the 1.3B-shaped layer (H=16, F=Dv=128, M=64) from a 32-token prefilled state,
    at the benchmark's batch sizes (both decode kernels: 16 and 256 slices take the
    row-parallel one, 1024 the mode-looping one)."""
    torch = _torch()
    ia = _lib()
    wl = W.decode(Bd, steps=4, prefix=32)
    pre, stp = wl["prefix"], wl["steps"]
    lam, beta = wl["lam"], wl["beta"]
    tag(f"decode 1.3b B={Bd} prefix")
    st = ia.new_state(Bd, 16, 64, 128, 128)
    ia.prefill(dev(pre["q"], torch.bfloat16), dev(pre["k"], torch.bfloat16),
               dev(pre["v"], torch.bfloat16), dev(lam), dev(beta), state=st, want_output=False)
    _, _, _, st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], lam, beta, threads=8)
    torch.cuda.synchronize()
    # the prefix state comes from bf16 inputs through the chunked MFMA path: bf16 tolerance
    err = state_rel(tuple(host(s) for s in st), st_ref)
    report(f"decode 1.3b B={Bd} prefix state", err)
    assert err < TOL_BF16
    for t in range(4):
        tag(f"decode 1.3b B={Bd} step {t}")
        o = ia.decode(dev(stp["q"][t], torch.bfloat16), dev(stp["k"][t], torch.bfloat16),
                      dev(stp["v"][t], torch.bfloat16), dev(lam), dev(beta), st)
        o_ref, st_ref = oracle.decode_step(stp["q"][t], stp["k"][t], stp["v"][t], lam, beta,
                                           st_ref)
        torch.cuda.synchronize()
        err = rowrel(host(o), o_ref)
        report(f"decode 1.3b B={Bd} step {t}", err)
        assert err < TOL_BF16


@pytest.mark.parametrize("shape", [(64, 32, 16), (16, 240, 48), (128, 64, 128), (256, 256, 128)])
def test_bf16_token_sequential_shapes(shape):
    """bf16 inputs on shapes the chunked kernels do not take (F != Dv, widths 240/256, M=128;
    256/256/128 is the largest the library accepts): prefill through the token-sequential
    kernel, then two decode steps (the mode-looping kernel), outputs and state.  The inputs
    are bf16-exact, so the oracle sees the same values and fp32 arithmetic sets the bar."""
    torch = _torch()
    ia = _lib()
    F, D, M = shape
    B, H, N = 2, 2, 37
    inp = W.make_inputs(B, H, N + 2, F, D, M, dtype="bf16", seed=F + 3 * D + 7 * M)
    lam, beta = inp["lam"], inp["beta"]
    q, k, v = (inp[n] for n in "qkv")
    bf = torch.bfloat16
    tag(f"bf16 token-sequential prefill F={F} D={D} M={M}")
    st = ia.new_state(B, H, M, F, D)
    o = ia.prefill(dev(q[:, :N], bf), dev(k[:, :N], bf), dev(v[:, :N], bf), dev(lam), dev(beta),
                   state=st, out_dtype=torch.float32)
    o_ref, _, _, st_ref = oracle.prefill(q[:, :N], k[:, :N], v[:, :N], lam, beta)
    torch.cuda.synchronize()
    err = rowrel(host(o), o_ref)
    report(f"bf16 token-sequential F={F} D={D} M={M} output", err)
    assert err < TOL_F32
    assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32
    st_ref = tuple(host(s) for s in st)   # both sides continue from the complex64 state
    for t in range(N, N + 2):
        tag(f"decode F={F} D={D} M={M} step {t - N}")
        o = ia.decode(dev(q[:, t], bf), dev(k[:, t], bf), dev(v[:, t], bf), dev(lam), dev(beta), st)
        o_ref, st_ref = oracle.decode_step(q[:, t], k[:, t], v[:, t], lam, beta, st_ref)
        torch.cuda.synchronize()
        assert rowrel(host(o), o_ref) < TOL_F32
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32
