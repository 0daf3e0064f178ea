"""GPU parity of the readout options against the oracle.

* IA_FLAG_NO_DEN: the output is the numerator alone, Re(phi(q) U^T Gamma) (the readout that
  drops the normaliser, summary page §3.1); the oracle returns that numerator beside o.
* IA_FLAG_IDENTITY_FEATURES: q and k are used as features as they stand.  The oracle has one
  feature map (elu + 1), so each case draws positive features f, hands f to the kernels and
  phi^-1(f) (f - 1 above 1, log f at or below it) to the oracle, whose phi then gives f back.

Every kernel family is covered: chunked MFMA prefill (bf16, both chunk lengths, the F=128 /
M=64 kernel, bidirectional), the fp32 token scan and both decode kernels.  Tolerances as
for the plain readout: row-wise relative 2e-3 with fp32 inputs, 2e-2 with bf16.
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


def _features(x, dtype):
    """Positive features of `dtype`-exact value: elu(x) + 1 rounded to the input type."""
    f = np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    f = W.round_bf16(f) if dtype == "bf16" else np.asarray(f, np.float32)
    return np.asarray(f, np.float64)


def _phi_inv(f):
    """The preimage of f > 0 under elu + 1."""
    return np.where(f > 1.0, f - 1.0, np.log(np.minimum(f, 1.0)))


def _identity_inputs(inp):
    """(kernel q, k; oracle q, k) for the identity-feature cases."""
    fq, fk = _features(inp["q"], inp["dtype"]), _features(inp["k"], inp["dtype"])
    return fq, fk, _phi_inv(fq), _phi_inv(fk)


def _prefill(inp, q=None, k=None, dtype="bf16", out="f32", **kw):
    import torch
    ia = _ia()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = inp["q"] if q is None else q
    k = inp["k"] if k is None else k
    od = torch.float32 if out == "f32" else torch.bfloat16
    o = ia.prefill(dev(q, td), dev(k, td), dev(inp["v"], td), dev(inp["lam"]),
                   dev(inp["beta"]), out_dtype=od, **kw)
    torch.cuda.synchronize()
    return o


def _flip(a):
    return np.ascontiguousarray(np.asarray(a)[:, ::-1])


@pytest.mark.parametrize("shape", [(2, 2, 200, 32, 16), (1, 3, 130, 64, 32),
                                   (1, 2, 257, 128, 64), (1, 2, 1, 64, 16)])
@pytest.mark.parametrize("chunk", [32, 64])
def test_no_den_chunk(shape, chunk):
    B, H, N, F, M = shape
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=300 + N + F + chunk)
    tag(f"no-den chunk prefill B={B} H={H} N={N} F={F} M={M} C={chunk}")
    o = _prefill(inp, chunk=chunk, no_den=True)
    num = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])[1]
    err = rowrel(host(o), num)
    report(f"no-den chunk {shape} C={chunk}", err)
    assert err < TOL_BF16


def test_no_den_chunk_state_and_bf16_output():
    """Non-zero initial state, many segments, bf16 output: the numerator and the final state
    (which the readout option leaves alone)."""
    B, H, N, F, M = 1, 2, 1500, 128, 64
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=311)
    pre = W.make_inputs(B, H, 16, F, F, M, dtype="bf16", seed=312)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    tag("no-den chunk prefill with state, bf16 out")
    o = _prefill(inp, out="bf16", state=st, no_den=True)
    _, num, _, st_out = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"],
                                       state=st_ref, threads=2)
    e_o, e_s = rowrel(host(o), num), state_rel(tuple(host(s) for s in st), st_out)
    report("no-den with state output", e_o)
    report("no-den with state state", e_s)
    assert e_o < TOL_BF16 and e_s < TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_den_bidirectional(dtype):
    B, H, N, F, M = 1, 2, 150, 64, 32
    inp = W.make_inputs(B, H, N, F, F, M, dtype=dtype, seed=320)
    tag(f"no-den bidir {dtype}")
    o = _prefill(inp, dtype=dtype, bidir=True, no_den=True)
    fwd = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])[1]
    rev = oracle.prefill(_flip(inp["q"]), _flip(inp["k"]), _flip(inp["v"]), inp["lam"],
                         inp["beta"])[1]
    err = rowrel(host(o), fwd + rev[:, ::-1])
    report(f"no-den bidir {dtype}", err)
    assert err < (TOL_BF16 if dtype == "bf16" else TOL_F32)


@pytest.mark.parametrize("N", [1, 77, 300])
def test_no_den_fp32_scan(N):
    B, H, F, D, M = 2, 2, 32, 48, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=330 + N)
    pre = W.make_inputs(B, H, 9, F, D, M, dtype="f32", seed=331, std=0.5)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    tag(f"no-den fp32 scan N={N}")
    o = _prefill(inp, dtype="f32", state=st, no_den=True)
    _, num, _, st_out = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"],
                                       state=st_ref)
    e_o, e_s = rowrel(host(o), num), state_rel(tuple(host(s) for s in st), st_out)
    report(f"no-den fp32 scan N={N}", e_o)
    assert e_o < TOL_F32 and e_s < TOL_F32


def _decode_case(B, H, F, D, M, dtype, steps, seed, identity):
    import torch
    ia = _ia()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = W.make_inputs(B, H, steps, F, D, M, dtype=dtype, seed=seed)
    lam, beta = inp["lam"], inp["beta"] * np.complex64(0.8 + 0.3j)
    pre = W.make_inputs(B, H, 9, F, D, M, dtype="f32", seed=seed + 1, std=0.5)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], lam, beta, threads=8)[3]
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    if identity:
        qk, kk, qo, ko = _identity_inputs(inp)
    else:
        qk, kk, qo, ko = inp["q"], inp["k"], inp["q"], inp["k"]
    for t in range(steps):
        tag(f"decode B={B} H={H} F={F} D={D} M={M} {dtype} identity={identity} step {t}")
        o = ia.decode(dev(qk[:, t], td), dev(kk[:, t], td), dev(inp["v"][:, t], td), dev(lam),
                      dev(beta), st, no_den=True, identity_features=identity)
        _, num, _, st_ref = oracle.prefill(qo[:, t:t + 1], ko[:, t:t + 1],
                                           inp["v"][:, t:t + 1], lam, beta, st_ref, threads=8)
        torch.cuda.synchronize()
        err = rowrel(host(o), num[:, 0])
        report(f"decode no-den step {t}", err)
        assert err < (TOL_BF16 if dtype == "bf16" else TOL_F32)
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("shape", [(2, 3, 32, 48, 16), (1, 16, 128, 128, 64),
                                   (64, 16, 128, 128, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_den_decode(shape, dtype):
    """Small shape (generic kernel), 16 slices (row-parallel kernel), 1024 slices (the
    mode-looping kernel) at F = Dv = 128, M = 64."""
    B, H, F, D, M = shape
    _decode_case(B, H, F, D, M, dtype, steps=3, seed=340 + B, identity=False)


@pytest.mark.parametrize("shape", [(2, 3, 32, 48, 16), (1, 16, 128, 128, 64)])
def test_identity_decode(shape):
    B, H, F, D, M = shape
    _decode_case(B, H, F, D, M, "f32", steps=3, seed=350 + B, identity=True)


@pytest.mark.parametrize("shape", [(2, 2, 200, 32, 16), (1, 2, 257, 128, 64)])
@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("no_den", [False, True])
def test_identity_chunk(shape, chunk, no_den):
    B, H, N, F, M = shape
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=360 + N + chunk)
    qk, kk, qo, ko = _identity_inputs(inp)
    tag(f"identity chunk prefill {shape} C={chunk} no_den={no_den}")
    o = _prefill(inp, q=qk, k=kk, chunk=chunk, identity_features=True, no_den=no_den)
    o_ref, num, _, _ = oracle.prefill(qo, ko, inp["v"], inp["lam"], inp["beta"])
    err = rowrel(host(o), num if no_den else o_ref)
    report(f"identity chunk {shape} C={chunk} no_den={no_den}", err)
    assert err < TOL_BF16


def test_identity_fp32_scan_with_state():
    import torch
    ia = _ia()
    B, H, N, F, D, M = 2, 2, 90, 32, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=370)
    qk, kk, qo, ko = _identity_inputs(inp)
    st = ia.new_state(B, H, M, F, D)
    tag("identity fp32 scan")
    o = _prefill(inp, q=qk, k=kk, dtype="f32", state=st, identity_features=True)
    o_ref, _, _, st_ref = oracle.prefill(qo, ko, inp["v"], inp["lam"], inp["beta"])
    torch.cuda.synchronize()
    assert rowrel(host(o), o_ref) < TOL_F32
    assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


def test_no_den_1p3b_workload_all_slices():
    """The 1.3B-shaped prefill (B=4, H=16, N=2048, F=Dv=128, M=64) in the benchmark's launch
    configuration, numerator readout, on every (b, h) slice."""
    wl = W.l1p3b()
    tag("no-den 1.3b workload")
    o = host(_prefill(wl, no_den=True))
    num = oracle.prefill(wl["q"], wl["k"], wl["v"], wl["lam"], wl["beta"], threads=16)[1]
    err = rowrel(o, num)
    report("no-den 1.3b, every slice", err)
    assert err < TOL_BF16
