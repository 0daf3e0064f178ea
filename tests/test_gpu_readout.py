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


def _R(H, M, seed, eps=0.3):
    rng = np.random.default_rng(seed)
    R = np.eye(M)[None] + eps * (rng.standard_normal((H, M, M))
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


# ---------------------------------------------------------------- chunked MFMA path (bf16)
# With bf16 inputs on the chunk kernels' shapes the readout matrix runs on the chunked path:
# a R formed per chunk on MFMA between the query-mode matrix and both readouts (chunk 64, or 32
# where the 64-token LDS layout has no room for R: F = Dv = 128 with M = 64).

def _worst(o, ref):
    B, H = o.shape[0], o.shape[2]
    errs = np.array([[rowrel(o[b, :, h], ref[b, :, h]) for h in range(H)] for b in range(B)])
    b, h = np.unravel_index(np.argmax(errs), errs.shape)
    return float(errs[b, h]), (int(b), int(h))


def _bf16_readout_run(inp, R, state=None, out="bf16", **kw):
    import torch
    ia = _ia()
    td = torch.bfloat16
    return ia.prefill(dev(inp["q"], td), dev(inp["k"], td), dev(inp["v"], td), dev(inp["lam"]),
                      dev(inp["beta"]), state=state,
                      out_dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                      readout=dev(R), **kw)


@pytest.mark.parametrize("name", ["125m", "1.3b"])
def test_readout_matrix_chunked_workload_all_slices(name):
    """The 125M and 1.3B workloads with a readout matrix per head, every (b, h) slice and the
    final state against scan_readout.  R = I + 0.05 (X + iY)/sqrt(M).  The bf16 operands'
    error is a few 2^-8 of the readout's terms, so the output error grows with the terms over
    the denominator, which the mixing R raises: at 0.3 some rows' oracle denominators turn
    negative (the clamp, not the layer, then decides the output), and at 0.1 one 1.3B head
    (dt = 0.03) reaches 2.8e-2."""
    import torch
    ia = _ia()
    inp = W.l125m() if name == "125m" else W.l1p3b()
    sh = inp["shape"]
    B, H, F, D, M = sh["B"], sh["H"], sh["F"], sh["D"], sh["M"]
    R = _R(H, M, 640, eps=0.05)
    st = ia.new_state(B, H, M, F, D)
    tag(f"readout matrix, chunked path: {name} workload, every slice and the final state")
    o = host(_bf16_readout_run(inp, R, state=st))
    torch.cuda.synchronize()
    o_ref, _, _, st_ref = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], inp["lam"],
                                                 inp["beta"], R, threads=16)
    worst, where = _worst(o, o_ref)
    report(f"readout matrix chunked {name} output (worst slice b,h={where})", worst)
    e_s = state_rel(tuple(host(s) for s in st), st_ref)
    report(f"readout matrix chunked {name} final state", e_s)
    assert worst < TOL_BF16 and e_s < TOL_BF16


@pytest.mark.parametrize("chunk", [0, 32, 64])
@pytest.mark.parametrize("shape", [(2, 3, 200, 32, 16), (1, 2, 333, 64, 64),
                                   (1, 2, 130, 128, 32), (1, 2, 161, 128, 64)])
def test_readout_matrix_chunked_shapes(shape, chunk):
    """Ragged lengths over several chunks and segments, both chunk lengths, with a caller state
    in and out; F = 128 with M = 64 has no 64-token instantiation and refuses chunk 64."""
    import torch
    ia = _ia()
    B, H, N, F, M = shape
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=650 + N)
    R = _R(H, M, 651)
    pre = W.make_inputs(B, H, 11, F, F, M, dtype="bf16", seed=652)
    st_ref0 = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
    st = tuple(dev(x) for x in st_ref0)
    st_ref0 = tuple(host(x) for x in st)
    tag(f"readout matrix chunked shape {shape} chunk={chunk}")
    if chunk == 64 and F == 128 and M == 64:
        with pytest.raises(RuntimeError, match="UNSUPPORTED"):
            _bf16_readout_run(inp, R, state=st, out="f32", chunk=chunk)
        return
    o = host(_bf16_readout_run(inp, R, state=st, out="f32", chunk=chunk))
    torch.cuda.synchronize()
    o_ref, _, _, st_ref = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], inp["lam"],
                                                 inp["beta"], R, state=st_ref0, threads=8)
    err = rowrel(o, o_ref)
    e_s = state_rel(tuple(host(x) for x in st), st_ref)
    report(f"readout matrix chunked {shape} chunk={chunk}", max(err, e_s))
    assert err < TOL_BF16 and e_s < TOL_BF16


def test_readout_matrix_chunked_bidirectional_no_den_and_route():
    """The genomic shape (F = Dv = M = 32) bidirectional with a readout matrix; the
    no-denominator readout; and a head whose modes the chunk factorisation does not resolve
    (dt = 0.3), which runs the fp32 recurrence with R inside the chunked launch."""
    import torch
    ia = _ia()
    B, H, N, F, M = 2, 2, 1500, 32, 32
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=660)
    R = _R(H, M, 661)
    fl = lambda a: np.ascontiguousarray(np.asarray(a)[:, ::-1])
    tag("readout matrix chunked bidirectional")
    o = host(_bf16_readout_run(inp, R, bidir=True))
    torch.cuda.synchronize()
    f = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], R,
                               threads=4)[0]
    r = oracle.prefill_readout(fl(inp["q"]), fl(inp["k"]), fl(inp["v"]), inp["lam"], inp["beta"],
                               R, threads=4)[0]
    err = _worst(o, f + r[:, ::-1])[0]
    report("readout matrix chunked bidir", err)
    assert err < TOL_BF16
    tag("readout matrix chunked no-den")
    o = host(_bf16_readout_run(inp, R, out="f32", no_den=True))
    torch.cuda.synchronize()
    num = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], R,
                                 threads=4)[1]
    err = _worst(o, num)[0]
    report("readout matrix chunked no-den", err)
    assert err < TOL_BF16
    lam = inp["lam"].copy()
    lam[1] = W.s4d_lin(np.array([0.3]), M)[0]
    inp["lam"] = lam
    assert ia.ia_check_lambda(ia.make_desc(B, H, N, F, F, M), lam) == 1
    tag("readout matrix chunked, head 1 on the fp32 route")
    o = host(_bf16_readout_run(inp, R, out="f32"))
    torch.cuda.synchronize()
    o_ref = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], lam, inp["beta"], R,
                                   threads=4)[0]
    e0, e1 = rowrel(o[:, :, 0], o_ref[:, :, 0]), rowrel(o[:, :, 1], o_ref[:, :, 1])
    report("readout matrix chunked head / routed head", max(e0, e1))
    assert e0 < TOL_BF16 and e1 < TOL_F32
