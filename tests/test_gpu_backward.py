"""GPU parity of the backward pass (ia_prefill_bwd) against the oracle's reverse-mode gradients
(``oracle.prefill_bwd``, pinned to the forward oracle by finite differences).

Error metric for gradients: slice-wise relative error, max over a (b,h) slice of
|x - ref| divided by the max of |ref| over that slice (a gradient row can be exactly zero,
e.g. dq at t = 0 from a zero state, so row-wise scaling would divide by nothing); for
dlambda and dbeta, per head over its modes.  Bounds: 2e-3 with fp32 inputs, 2e-2 with bf16
inputs and outputs.
"""
import numpy as np
import pytest

import ia_workloads as W
import oracle
from helpers import TOL_BF16, TOL_F32, dev, host, report, tag

pytestmark = pytest.mark.gpu


def _ia():
    import ssm_sequence_mixer_amd as ia
    return ia


def slice_rel(x, ref, slices=None):
    """max over (b,h) slices of max|x - ref| / max|ref| within the slice ([B,N,H,X] arrays)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    B, _, H, _ = ref.shape
    worst = 0.0
    for b, h in slices or [(b, h) for b in range(B) for h in range(H)]:
        r = ref[b, :, h]
        e = np.max(np.abs(x[b, :, h] - r)) / max(np.max(np.abs(r)), 1e-300)
        worst = max(worst, float(e) if np.isfinite(e) else np.inf)
    return worst


def head_rel(x, ref):
    """max over heads of max|x - ref| / max|ref| over the head's modes ([H,M] complex)."""
    x, ref = np.asarray(x), np.asarray(ref)
    return max(float(np.max(np.abs(x[h] - ref[h])) / max(np.max(np.abs(ref[h])), 1e-300))
               for h in range(ref.shape[0]))


def state_rel(st, ref):
    out = []
    for a, b in zip(st, ref):
        a = np.asarray(a).reshape(a.shape[0], a.shape[1], -1)
        b = np.asarray(b).reshape(b.shape[0], b.shape[1], -1)
        scale = np.maximum(np.max(np.abs(b), axis=-1), 1e-300)
        out.append(float(np.max(np.max(np.abs(a - b), axis=-1) / scale)))
    return max(out)


def _run(inp, dO, dtype="f32", state=None, want_state=False, **kw):
    import torch
    ia = _ia()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (dev(inp[n], td) for n in "qkv")
    st = None if state is None else tuple(dev(s) for s in state)
    r = ia.prefill_bwd(q, k, v, dev(inp["lam"]), dev(inp["beta"]), dev(dO), state0=st,
                       want_state_grad=want_state, **kw)
    torch.cuda.synchronize()
    dq, dk, dv, dl, db, dst = r
    return (host(dq), host(dk), host(dv), host(dl), host(db),
            None if dst is None else tuple(host(s) for s in dst))


def _compare(got, ref, tol, name, slices=None, state=False):
    dq, dk, dv, dl, db, dst = got
    rq, rk, rv, rl, rb, rst = ref
    errs = {"dq": slice_rel(dq, rq, slices), "dk": slice_rel(dk, rk, slices),
            "dv": slice_rel(dv, rv, slices)}
    if slices is None:
        errs["dlam"] = head_rel(dl, rl.sum(axis=0))
        errs["dbeta"] = head_rel(db, rb.sum(axis=0))
    if state:
        errs["dstate0"] = state_rel(dst, rst)
    for k, e in errs.items():
        report(f"{name} {k}", e)
    assert max(errs.values()) < tol, errs


# Shapes with F == Dv in {32, 64, 128} run the chunked MFMA backward on the automatic path (these
# sequences are short); path="sequential" asks for the token-sequential kernels, which the other
# shapes always run.
@pytest.mark.parametrize("path", ["auto", "sequential"])
@pytest.mark.parametrize("shape", [
    (2, 2, 70, 32, 32, 16), (1, 2, 100, 64, 48, 16), (1, 1, 97, 128, 128, 64),
    (1, 2, 65, 16, 16, 32), (2, 1, 33, 32, 32, 16), (2, 1, 64, 256, 64, 16),
    (1, 1, 40, 192, 256, 32), (2, 2, 48, 64, 64, 48), (1, 3, 16, 32, 32, 32)])
def test_backward_fp32_matches_oracle(shape, path):
    B, H, N, F, D, M = shape
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=500 + N + F + D + M)
    dO = np.random.default_rng(501 + N).standard_normal((B, N, H, D)).astype(np.float32)
    tag(f"backward fp32 B={B} H={H} N={N} F={F} D={D} M={M} path={path}")
    got = _run(inp, dO, path=path)
    ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO,
                             threads=4)
    _compare(got, ref, TOL_F32, f"bwd {shape} path={path}")


@pytest.mark.parametrize("FD", [(64, 32), (64, 64)])
@pytest.mark.parametrize("N", [1, 2, 15, 16, 17, 31, 32, 33, 200])
def test_backward_with_initial_state(N, FD):
    """Non-zero initial state; the gradient of the initial state too; N around the
    checkpoint interval and the chunk length (F = Dv = 64 runs the chunked kernels, 64/32 the
    token-sequential ones).  (The first few tokens from a zero state are tested here, from a
    state, and in absolute terms below: from zero, o_t for t < 3 or so hardly depends on q
    and k, so their gradients are small differences of the numerator's and denominator's
    terms, and fp32 rounding of those terms is not small relative to them.)"""
    B, H, M = 1, 2, 32
    F, D = FD
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=510 + N)
    pre = W.make_inputs(B, H, 12, F, D, M, dtype="f32", seed=511, std=0.5)
    st = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
    st = tuple(np.asarray(s, np.complex64).astype(np.complex128) for s in st)
    dO = np.random.default_rng(512).standard_normal((B, N, H, D)).astype(np.float32)
    tag(f"backward with state N={N} F={F} D={D}")
    got = _run(inp, dO, state=st, want_state=True)
    ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO,
                             state=st)
    _compare(got, ref, TOL_F32, f"bwd state N={N} F={F} D={D}", state=True)


def test_backward_single_token_from_zero_state():
    """One token from a zero state gives o = v whatever q, k and beta are: their gradients
    vanish (up to rounding) and dv = dO."""
    B, H, N, F, D, M = 2, 2, 1, 32, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=515)
    dO = np.random.default_rng(516).standard_normal((B, N, H, D)).astype(np.float32)
    tag("backward single token")
    dq, dk, dv, dl, db, _ = _run(inp, dO)
    assert np.max(np.abs(dv - dO)) < 1e-5 * np.max(np.abs(dO))
    assert np.max(np.abs(dq)) < 1e-4 and np.max(np.abs(dk)) < 1e-4
    assert np.max(np.abs(db)) < 1e-4 * np.max(np.abs(dO)) * B


def test_backward_without_denominator_and_identity_features():
    B, H, N, F, D, M = 1, 2, 90, 32, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=520)
    dO = np.random.default_rng(521).standard_normal((B, N, H, D)).astype(np.float32)
    tag("backward no-den")
    got = _run(inp, dO, no_den=True)
    ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO,
                             no_den=True)
    _compare(got, ref, TOL_F32, "bwd no-den")
    # identity features: the kernels take f, the oracle phi^-1(f); its dq is then
    # dL/df * phi'(phi^-1(f)) = dL/df * min(f, 1)
    fq = np.where(inp["q"] > 0, inp["q"] + 1, np.exp(np.minimum(inp["q"], 0))).astype(np.float32)
    fk = np.where(inp["k"] > 0, inp["k"] + 1, np.exp(np.minimum(inp["k"], 0))).astype(np.float32)
    fq64, fk64 = fq.astype(np.float64), fk.astype(np.float64)
    inv = lambda f: np.where(f > 1.0, f - 1.0, np.log(np.minimum(f, 1.0)))
    tag("backward identity features")
    got = _run({**inp, "q": fq, "k": fk}, dO, identity_features=True)
    ref = list(oracle.prefill_bwd(inv(fq64), inv(fk64), inp["v"], inp["lam"], inp["beta"], dO))
    ref[0] = ref[0] / np.where(fq64 > 1.0, 1.0, fq64)
    ref[1] = ref[1] / np.where(fk64 > 1.0, 1.0, fk64)
    _compare(got, tuple(ref), TOL_F32, "bwd identity")


def test_backward_clamped_denominator():
    """beta = i with real lambda puts every den below the clamp: den has no gradient."""
    B, H, N, F, D, M = 1, 1, 50, 32, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=530)
    lam = np.abs(inp["lam"]).astype(np.complex64)
    beta = np.full((H, M), 1j, np.complex64)
    inp = {**inp, "lam": lam, "beta": beta}
    den = oracle.prefill(inp["q"], inp["k"], inp["v"], lam, beta)[2]
    assert np.nanmax(den) < 0
    dO = np.random.default_rng(531).standard_normal((B, N, H, D)).astype(np.float32)
    tag("backward clamped")
    got = _run(inp, dO)
    ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], lam, beta, dO)
    _compare(got, ref, TOL_F32, "bwd clamped")


def test_backward_bf16_inputs():
    B, H, N, F, D, M = 2, 2, 150, 64, 64, 32
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=540)
    dO = W.round_bf16(np.random.default_rng(541).standard_normal((B, N, H, D)))
    import torch
    ia = _ia()
    tag("backward bf16")
    q, k, v = (dev(inp[n], torch.bfloat16) for n in "qkv")
    r = ia.prefill_bwd(q, k, v, dev(inp["lam"]), dev(inp["beta"]), dev(dO, torch.bfloat16))
    torch.cuda.synchronize()
    got = tuple(host(x) for x in r[:5]) + (None,)
    ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO,
                             threads=4)
    _compare(got, ref, TOL_BF16, "bwd bf16")


def test_backward_1p3b_workload_sampled():
    """The 1.3B-shaped layer (B=4, H=16, N=2048, F=Dv=128, M=64, bf16 q, k, v, fp32 dO), as
    the benchmark times it; one head's slices in full (its lambda, beta gradients are their
    sum over b) and one more slice."""
    import torch
    ia = _ia()
    wl = W.l1p3b()
    B, N, H = 4, 2048, 16
    dO = np.random.default_rng(550).standard_normal((B, N, H, 128)).astype(np.float32)
    tag("backward 1.3b workload")
    q, k, v = (dev(wl[n], torch.bfloat16) for n in "qkv")
    r = ia.prefill_bwd(q, k, v, dev(wl["lam"]), dev(wl["beta"]), dev(dO))
    torch.cuda.synchronize()
    got = tuple(host(x) for x in r[:5])
    slices = [(b, 5) for b in range(B)] + [(2, 11)]
    ref = oracle.prefill_bwd(wl["q"], wl["k"], wl["v"], wl["lam"], wl["beta"], dO,
                             slices=slices, threads=5)
    errs = {n: slice_rel(got[i], ref[i], slices) for i, n in enumerate(("dq", "dk", "dv"))}
    errs["dlam h=5"] = head_rel(got[3][5:6], ref[3][:, 5:6].sum(axis=0))
    errs["dbeta h=5"] = head_rel(got[4][5:6], ref[4][:, 5:6].sum(axis=0))
    for n, e in errs.items():
        report(f"bwd 1.3b {n}", e)
    assert max(errs.values()) < TOL_BF16, errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_bidirectional(dtype):
    """The bidirectional layer (both directions from zero): the causal gradients plus those of
    the reversed walk, against oracle.bidir_bwd."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 2, 2, 77, 32, 32, 32
    inp = W.make_inputs(B, H, N, F, D, M, dtype=dtype, seed=560)
    dO = np.random.default_rng(561).standard_normal((B, N, H, D)).astype(np.float32)
    if dtype == "bf16":
        dO = W.round_bf16(dO)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    tag(f"backward bidirectional {dtype}")
    q, k, v = (dev(inp[n], td) for n in "qkv")
    r = ia.prefill_bwd(q, k, v, dev(inp["lam"]), dev(inp["beta"]), dev(dO, td), bidir=True)
    torch.cuda.synchronize()
    got = tuple(host(x) for x in r[:5]) + (None,)
    ref = oracle.bidir_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO, threads=4)
    _compare(got, tuple(ref) + (None,), TOL_BF16 if dtype == "bf16" else TOL_F32,
             f"bwd bidir {dtype}")


@pytest.mark.parametrize("path", ["sequential", "chunked"])
@pytest.mark.parametrize("case", ["state_fp32", "bf16", "bidir_fp32", "noden_fp32"])
def test_backward_sequence_segments(case, path):
    """Few slices and long enough sequences that the token-sequential sweeps are cut into
    segments of 256+ tokens (1000 or 2000 tokens: 4 to 8 segments, the last one ragged), joined
    by the state and adjoint carries; with path="chunked" the same long sequences on the
    chunked kernels (one walk per slice and mode group, F = Dv)."""
    import torch
    ia = _ia()
    dtype = "bf16" if case == "bf16" else "f32"
    B, H, N, F, D, M = (1, 2, 2000, 64, 32, 32) if case == "bf16" else (1, 2, 1000, 32, 32, 16)
    if path == "chunked" and case == "bf16":
        D = 64
    inp = W.make_inputs(B, H, N, F, D, M, dtype=dtype, seed=570 + N)
    dO = np.random.default_rng(571).standard_normal((B, N, H, D)).astype(np.float32)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    st = None
    if case == "state_fp32":
        pre = W.make_inputs(B, H, 12, F, D, M, dtype="f32", seed=572, std=0.5)
        st = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
        st = tuple(np.asarray(x, np.complex64).astype(np.complex128) for x in st)
    tag(f"backward segments {case} N={N} path={path}")
    q, k, v = (dev(inp[n], td) for n in "qkv")
    r = ia.prefill_bwd(q, k, v, dev(inp["lam"]), dev(inp["beta"]), dev(dO),
                       state0=None if st is None else tuple(dev(x) for x in st),
                       want_state_grad=st is not None, bidir=case == "bidir_fp32",
                       no_den=case == "noden_fp32", path=path)
    torch.cuda.synchronize()
    got = tuple(host(x) for x in r[:5]) + (None if r[5] is None else tuple(host(x) for x in r[5]),)
    if case == "bidir_fp32":
        ref = tuple(oracle.bidir_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO,
                                     threads=2)) + (None,)
    else:
        ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO,
                                 state=st, no_den=case == "noden_fp32", threads=2)
    _compare(got, ref, TOL_BF16 if dtype == "bf16" else TOL_F32,
             f"bwd segments {case} path={path}", state=st is not None)


@pytest.mark.parametrize("shape,dtype", [((1, 1, 40, 256, 256, 128), "f32"),
                                         ((2, 1, 70, 256, 128, 128), "bf16"),
                                         ((1, 2, 33, 16, 256, 16), "f32")])
def test_backward_largest_sizes(shape, dtype):
    """The largest F, Dv and M the boundary takes (the widest staged rows: blocks of 3 tokens),
    and the narrowest F beside the widest Dv."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = shape
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = W.make_inputs(B, H, N, F, D, M, dtype=dtype, seed=580 + F + M)
    dO = np.random.default_rng(581).standard_normal((B, N, H, D)).astype(np.float32)
    tag(f"backward largest sizes {shape} {dtype}")
    q, k, v = (dev(inp[n], td) for n in "qkv")
    r = ia.prefill_bwd(q, k, v, dev(inp["lam"]), dev(inp["beta"]), dev(dO))
    torch.cuda.synchronize()
    got = tuple(host(x) for x in r[:5]) + (None,)
    ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO,
                             threads=2)
    _compare(got, ref, TOL_BF16 if dtype == "bf16" else TOL_F32, f"bwd largest {shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_chunked_128_modes(dtype):
    """M = 128 with F = Dv = 128 on the chunked kernels: eight groups of 16 modes, the most the
    per-token den partials of a chunk are summed over, and a ragged last chunk."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 1, 2, 45, 128, 128, 128
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp = W.make_inputs(B, H, N, F, D, M, dtype=dtype, seed=590)
    dO = np.random.default_rng(591).standard_normal((B, N, H, D)).astype(np.float32)
    tag(f"backward chunked M=128 {dtype}")
    q, k, v = (dev(inp[n], td) for n in "qkv")
    r = ia.prefill_bwd(q, k, v, dev(inp["lam"]), dev(inp["beta"]), dev(dO), path="chunked")
    torch.cuda.synchronize()
    got = tuple(host(x) for x in r[:5]) + (None,)
    ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], dO,
                             threads=2)
    _compare(got, ref, TOL_BF16 if dtype == "bf16" else TOL_F32, f"bwd chunked M=128 {dtype}")


@pytest.mark.parametrize("mag,no_den", [(1.0, False), (0.5, False), (0.5, True), (0.1, True),
                                         (0.01, True)])
def test_backward_chunked_lambda_magnitudes(mag, no_den):
    """Modes of one magnitude on the chunked kernels, fp32: undamped (|lambda| = 1, the S4D-Lin
    angles of dt = 0.01) and fast-decaying ones down to |lambda| = 0.01, where the chunk-local
    powers lambda^e (|e| <= 9) span 1e-16 to 1e18.  Below |lambda| ~ 0.5 the normalised
    readout is the plain-definition limit o_t -> v_t: dq and dk become differences of the
    numerator's and the denominator's terms that cancel to 1e-7 of their size (the fp64 oracle
    itself holds them to about 1e-11), so those magnitudes run the readout without the
    denominator, whose gradients do not cancel."""
    B, H, N, F, D, M = 2, 2, 70, 32, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=600)
    if mag == 1.0:
        ang = np.pi * 0.01 * np.arange(M)[None, :].repeat(H, 0)
    else:
        ang = np.random.default_rng(601).uniform(-np.pi, np.pi, (H, M))
    lam = (mag * np.exp(1j * ang)).astype(np.complex64)
    inp = {**inp, "lam": lam}
    dO = np.random.default_rng(602).standard_normal((B, N, H, D)).astype(np.float32)
    tag(f"backward chunked |lambda|={mag} no_den={no_den}")
    got = _run(inp, dO, path="chunked", no_den=no_den)
    ref = oracle.prefill_bwd(inp["q"], inp["k"], inp["v"], lam, inp["beta"], dO, no_den=no_den,
                             threads=2)
    _compare(got, ref, TOL_F32, f"bwd chunked |lambda|={mag} no_den={no_den}")
