"""GPU parity of the readout-matrix variants (ia_prefill_fwd_readout, ia_decode_step_readout)
against the oracle's ``scan_readout``, which the brute-force double sum and the R = I and
linearity pins tie down.  The readouts use a R in place of a (R a learned complex M x M
matrix per head).  Tolerances: row-wise relative 2e-3 with fp32 inputs, 2e-2 with bf16.
"""
import numpy as np
import pytest

import ia_workloads as W
import oracle
from helpers import TOL_BF16, TOL_F32, dev, host, report, rowrel, state_rel, tag

pytestmark = pytest.mark.gpu


def _ia():
    import ssm_sequence_mixer_amd as ia
    return ia


def _R(H, M, seed):
    rng = np.random.default_rng(seed)
    R = np.eye(M)[None] + 0.3 * (rng.standard_normal((H, M, M))
                                 + 1j * rng.standard_normal((H, M, M))) / np.sqrt(M)
    return R.astype(np.complex64).astype(np.complex128)


@pytest.mark.parametrize("shape", [(2, 3, 32, 48, 16), (1, 16, 128, 128, 64),
                                   (64, 16, 128, 128, 64), (2, 2, 64, 64, 128),
                                   (1, 2, 256, 256, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_readout_matrix(shape, dtype):
    """Generic kernel, row-parallel kernel (16 slices) and mode-looping kernel (1024 slices),
    and the largest mode count (M = 128) on both kernels."""
    import torch
    ia = _ia()
    B, H, F, D, M = shape
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = W.make_inputs(B, H, 3, F, D, M, dtype=dtype, seed=600 + B)
    lam, beta = inp["lam"], inp["beta"]
    R = _R(H, M, 601)
    pre = W.make_inputs(B, H, 9, F, D, M, dtype="f32", seed=602, std=0.5)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], lam, beta, threads=8)[3]
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    Rd = dev(R)
    for t in range(3):
        tag(f"decode readout matrix B={B} H={H} F={F} D={D} M={M} {dtype} step {t}")
        o = ia.decode(dev(inp["q"][:, t], td), dev(inp["k"][:, t], td), dev(inp["v"][:, t], td),
                      dev(lam), dev(beta), st, readout=Rd)
        o_ref, _, _, st_ref = oracle.prefill_readout(inp["q"][:, t:t + 1], inp["k"][:, t:t + 1],
                                                     inp["v"][:, t:t + 1], lam, beta, R, st_ref,
                                                     threads=8)
        torch.cuda.synchronize()
        err = rowrel(host(o), o_ref[:, 0])
        report(f"decode readout {shape} {dtype} step {t}", err)
        assert err < (TOL_BF16 if dtype == "bf16" else TOL_F32)
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_state", [False, True])
def test_prefill_readout_matrix(dtype, with_state):
    import torch
    ia = _ia()
    B, H, N, F, D, M = 2, 2, 130, 64, 64, 32
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = W.make_inputs(B, H, N, F, D, M, dtype=dtype, seed=610)
    R = _R(H, M, 611)
    st_ref = None
    st = None
    if with_state:
        pre = W.make_inputs(B, H, 9, F, D, M, dtype="f32", seed=612, std=0.5)
        st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
        st = tuple(dev(s) for s in st_ref)
        st_ref = tuple(host(s) for s in st)
    tag(f"prefill readout matrix {dtype} state={with_state}")
    o = ia.prefill(dev(inp["q"], td), dev(inp["k"], td), dev(inp["v"], td), dev(inp["lam"]),
                   dev(inp["beta"]), state=st, out_dtype=torch.float32, readout=dev(R))
    torch.cuda.synchronize()
    o_ref, _, _, st_out = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], inp["lam"],
                                                 inp["beta"], R, st_ref, threads=4)
    err = rowrel(host(o), o_ref)
    report(f"prefill readout {dtype} state={with_state}", err)
    assert err < (TOL_BF16 if dtype == "bf16" else TOL_F32)
    if with_state:
        assert state_rel(tuple(host(s) for s in st), st_out) < TOL_F32


def test_prefill_readout_matrix_bidirectional_and_no_den():
    import torch
    ia = _ia()
    B, H, N, F, D, M = 1, 2, 70, 32, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=620)
    R = _R(H, M, 621)
    fl = lambda a: np.ascontiguousarray(np.asarray(a)[:, ::-1])
    tag("prefill readout matrix bidirectional")
    o = ia.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["lam"]), dev(inp["beta"]),
                   out_dtype=torch.float32, bidir=True, readout=dev(R))
    torch.cuda.synchronize()
    f = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], R)[0]
    r = oracle.prefill_readout(fl(inp["q"]), fl(inp["k"]), fl(inp["v"]), inp["lam"], inp["beta"],
                               R)[0]
    err = rowrel(host(o), f + r[:, ::-1])
    report("prefill readout bidir", err)
    assert err < TOL_F32
    tag("prefill readout matrix no-den")
    o = ia.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["lam"]), dev(inp["beta"]),
                   out_dtype=torch.float32, no_den=True, readout=dev(R))
    torch.cuda.synchronize()
    num = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], R)[1]
    err = rowrel(host(o), num)
    report("prefill readout no-den", err)
    assert err < TOL_F32


def test_readout_identity_matches_plain_call():
    """R = I through the readout entry point equals the plain fp32 token-sequential path."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 1, 2, 50, 32, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=630)
    eye = np.broadcast_to(np.eye(M, dtype=np.complex64), (H, M, M)).copy()
    tag("prefill readout identity")
    args = (dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["lam"]), dev(inp["beta"]))
    o1 = ia.prefill(*args, out_dtype=torch.float32, readout=dev(eye))
    o2 = ia.prefill(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rowrel(host(o1), host(o2)) < 1e-5
