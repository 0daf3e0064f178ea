"""GPU parity of selective writing and memory decay (ia_prefill_fwd_gated, ia_decode_step_gated)
against the oracle's gated recurrence (oracle.scan_gated, pinned in tests/test_oracle.py).

bf16 inputs on the chunk kernels' shapes run the chunked MFMA prefill with the gates folded in
(the bf16 bound); fp32 inputs, and bf16 inputs on other shapes, run the token-sequential fp32
kernels (the inputs reach both sides as the same numbers: the fp32 bound).  Gates: write gates
in (0, 1.5), decay gates in (0.5, 1], and on the chunked path also negative and zero gates.

Where a row's readout sums cancel, bf16 operands resolve the row only to about kappa 2^-9,
kappa = kappa_den + kappa_num of oracle.brute.gated_condition (every term of the sums expanded
over key pairs and modes).  Rows above the bf16 bound are therefore held to 2 kappa 2^-9; rows
whose denominator is not resolved at all (4 kappa_den 2^-9 >= 1: its sign may flip against the
one-sided clamp) are exempt; and at most one row in twenty may be above the bound."""
import numpy as np
import pytest

import ia_workloads as W
import oracle
from oracle import brute
from helpers import TOL_BF16, TOL_F32, dev, host, report, rowrel, state_rel, tag

pytestmark = pytest.mark.gpu

BF16_EPS = 2.0 ** -9   # unit roundoff of bf16


def _ia():
    import ssm_sequence_mixer_amd as ia
    return ia


def _gates(rng, shape):
    return (rng.uniform(0.0, 1.5, shape).astype(np.float32),
            rng.uniform(0.5, 1.0, shape).astype(np.float32))


def _mild_gates(rng, shape):
    """Gates of a trained model's typical range: writes in [0.5, 1), decays in [0.9, 1)."""
    return (rng.uniform(0.5, 1.0, shape).astype(np.float32),
            rng.uniform(0.9, 1.0, shape).astype(np.float32))


def _chunked(dtype, F, D, M):
    """bf16 inputs on a shape the chunk kernels take."""
    return dtype == "bf16" and F == D and F in (32, 64, 128) and M in (16, 32, 64)


def _check_bf16_rows(o, o_ref, inp, wg, dg, label, state=None):
    """The bf16 bound per row, or, for rows above it, 2 kappa 2^-9 (module docstring)."""
    err = np.max(np.abs(o - o_ref), axis=-1) / np.maximum(np.max(np.abs(o_ref), axis=-1), 1e-30)
    assert not np.any(np.isnan(o) != np.isnan(o_ref))
    over = np.argwhere(err >= TOL_BF16)
    report(f"{label}: rows within the bf16 bound", float(np.max(np.where(err < TOL_BF16, err, 0.0))))
    cond, unresolved, worst = {}, 0, 0.0
    for b, h in {(int(b), int(h)) for b, _, h in over}:
        st = None if state is None else tuple(x[b, h] for x in state)
        rows = [n for bb, n, hh in over if bb == b and hh == h]
        cond[(b, h)] = brute.gated_condition(inp["q"][b, :, h], inp["k"][b, :, h],
                                             inp["v"][b, :, h], inp["lam"][h], inp["beta"][h],
                                             wg[b, :, h], dg[b, :, h], st, tokens=rows)
    for b, n, h in over:
        kd, kn = cond[(int(b), int(h))]
        if 4 * kd[n] * BF16_EPS >= 1:
            unresolved += 1
            continue
        ratio = err[b, n, h] / ((kd[n] + kn[n]) * BF16_EPS)
        worst = max(worst, ratio)
        assert ratio < 2, (b, n, h, err[b, n, h], kd[n], kn[n])
    report(f"{label}: {len(over)} rows above the bound ({unresolved} unresolved), "
           f"worst err / (kappa 2^-9)", worst)
    assert len(over) <= err.size // 20, len(over)


def _flip(a):
    return np.ascontiguousarray(np.asarray(a)[:, ::-1])


@pytest.mark.parametrize("shape", [(2, 3, 150, 32, 16, 16), (1, 2, 300, 64, 64, 32),
                                   (2, 2, 97, 128, 128, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_prefill_matches_oracle(shape, dtype):
    import torch
    ia = _ia()
    B, H, N, F, D, M = shape
    inp = W.make_inputs(B, H, N, F, D, M, dtype=dtype, seed=1000 + N + F)
    wg, dg = _gates(np.random.default_rng(1001 + N), (B, N, H))
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    pre = W.make_inputs(B, H, 7, F, D, M, dtype="f32", seed=1002, std=0.5)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
    st = tuple(dev(x) for x in st_ref)
    st_ref = tuple(host(x) for x in st)
    tag(f"gated prefill {shape} {dtype}")
    o = ia.prefill(dev(inp["q"], td), dev(inp["k"], td), dev(inp["v"], td), dev(inp["lam"]),
                   dev(inp["beta"]), state=st, out_dtype=torch.float32,
                   gates=(dev(wg), dev(dg)))
    torch.cuda.synchronize()
    o_ref, _, _, st_out = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"],
                                               inp["beta"], wg, dg, state=st_ref, threads=8)
    e_s = state_rel(tuple(host(x) for x in st), st_out)
    if _chunked(dtype, F, D, M):
        _check_bf16_rows(host(o), o_ref, inp, wg, dg, f"gated prefill {shape} bf16", st_ref)
        report(f"gated prefill {shape} bf16 state", e_s)
        assert e_s < TOL_BF16
        return
    e_o = rowrel(host(o), o_ref)
    report(f"gated prefill {shape} {dtype} output / state", max(e_o, e_s))
    assert e_o < TOL_F32 and e_s < TOL_F32


def test_gated_unit_gates_equal_the_plain_fp32_prefill():
    """Gates of one give the ungated fp32 prefill bit for bit (the same kernel, times 1)."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 2, 2, 120, 32, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=1010)
    args = [dev(inp[n]) for n in "qkv"] + [dev(inp["lam"]), dev(inp["beta"])]
    ones = torch.ones((B, N, H), dtype=torch.float32, device="cuda")
    tag("gated prefill, unit gates")
    o1 = ia.prefill(*args, gates=(ones, ones))
    o2 = ia.prefill(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("shape", [(1, 2, 60, 32, 32, 16), (2, 2, 97, 128, 128, 64),
                                   (1, 2, 300, 64, 64, 32)])
@pytest.mark.parametrize("kind", ["negative decay", "negative write", "zero decay"])
def test_gated_chunked_signed_and_zero_gates(shape, kind):
    """The chunked path with decay gates of either sign (the records carry the sign of each
    running product), negative write gates, and decay gates of exactly zero (|a| < 2^-64
    counts as 2^-64 there: the carried state drops to 2^-64 of itself instead of to zero),
    against the oracle's exact recurrence; one chunk, two segments (one slot), and many."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = shape
    sh = (B, N, H)
    rng = np.random.default_rng(1050 + N + len(kind))
    wg = rng.uniform(0.0, 1.5, sh).astype(np.float32)
    dg = rng.uniform(0.5, 1.0, sh).astype(np.float32)
    if kind == "negative decay":
        dg *= np.where(rng.uniform(size=sh) < 0.5, -1.0, 1.0).astype(np.float32)
    elif kind == "negative write":
        wg = rng.uniform(-1.0, 1.5, sh).astype(np.float32)
    else:
        dg[rng.uniform(size=sh) < 0.05] = 0.0
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=1051 + N)
    st = ia.new_state(B, H, M, F, D)
    tag(f"gated chunked prefill {shape} {kind}")
    o = ia.prefill(*(dev(inp[n], torch.bfloat16) for n in "qkv"), dev(inp["lam"]),
                   dev(inp["beta"]), state=st, out_dtype=torch.float32,
                   gates=(dev(wg), dev(dg)))
    torch.cuda.synchronize()
    o_ref, _, _, st_ref = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"],
                                               inp["beta"], wg, dg, threads=8)
    _check_bf16_rows(host(o), o_ref, inp, wg, dg, f"gated chunked {shape} {kind}")
    e_s = state_rel(tuple(host(x) for x in st), st_ref)
    report(f"gated chunked {shape} {kind} state", e_s)
    assert e_s < TOL_BF16


def test_gated_unit_gates_equal_the_plain_chunked_prefill():
    """Gates of one on the chunked path give the ungated chunked prefill up to the rounding
    of the two eta updates (a Horner sum over the chunk's end factors in place of the table's
    geometric sum); every other gate factor is exactly 1."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 2, 4, 1000, 128, 128, 64
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=1060)
    args = [dev(inp[n], torch.bfloat16) for n in "qkv"] + [dev(inp["lam"]), dev(inp["beta"])]
    ones = torch.ones((B, N, H), dtype=torch.float32, device="cuda")
    s1, s2 = ia.new_state(B, H, M, F, D), ia.new_state(B, H, M, F, D)
    tag("gated chunked prefill, unit gates")
    o1 = ia.prefill(*args, state=s1, out_dtype=torch.float32, gates=(ones, ones))
    o2 = ia.prefill(*args, state=s2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    e = max(rowrel(host(o1), host(o2)),
            state_rel(tuple(host(x) for x in s1), tuple(host(x) for x in s2)))
    report("gated chunked prefill, unit gates vs ungated", e)
    assert e < 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_decode_steps_continue_the_prefill(dtype):
    """A gated prefill of the first tokens, then gated decode steps (row-parallel kernel at
    these sizes, mode-looping at F = 256), equal the oracle's gated recurrence over all
    tokens, outputs and final state (the bf16 bound after a chunked prefill)."""
    import torch
    ia = _ia()
    for (B, H, F, D, M) in [(2, 4, 128, 128, 64), (1, 2, 256, 48, 32)]:
        N0, steps = 20, 5
        inp = W.make_inputs(B, H, N0 + steps, F, D, M, dtype=dtype, seed=1020 + F)
        wg, dg = _gates(np.random.default_rng(1021 + F), (B, N0 + steps, H))
        td = torch.float32 if dtype == "f32" else torch.bfloat16
        st = ia.new_state(B, H, M, F, D)
        tag(f"gated prefill then decode B={B} H={H} F={F} D={D} M={M} {dtype}")
        ia.prefill(*(dev(inp[n][:, :N0], td) for n in "qkv"), dev(inp["lam"]), dev(inp["beta"]),
                   state=st, want_output=False,
                   gates=(dev(wg[:, :N0]), dev(dg[:, :N0])))
        outs = []
        for t in range(N0, N0 + steps):
            outs.append(host(ia.decode(*(dev(inp[n][:, t], td) for n in "qkv"), dev(inp["lam"]),
                                       dev(inp["beta"]), st,
                                       gates=(dev(wg[:, t]), dev(dg[:, t])))))
        torch.cuda.synchronize()
        o_ref, _, _, st_ref = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"],
                                                   inp["beta"], wg, dg, threads=8)
        e_o = rowrel(np.stack(outs, axis=1), o_ref[:, N0:])
        e_s = state_rel(tuple(host(x) for x in st), st_ref)
        report(f"gated decode F={F} {dtype} outputs / state", max(e_o, e_s))
        tol = TOL_BF16 if _chunked(dtype, F, D, M) else TOL_F32   # the prefill's path
        assert e_o < tol and e_s < tol


def test_gated_bidirectional():
    """Both directions with the gates of the positions they walk: o = IA_g(x) +
    flip(IA_{flip g}(flip x)) (the chunked path: the bf16 bound)."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 1, 3, 211, 32, 32, 32
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=1030)
    wg, dg = _gates(np.random.default_rng(1031), (B, N, H))
    tag("gated bidirectional prefill")
    o = ia.prefill(*(dev(inp[n], torch.bfloat16) for n in "qkv"), dev(inp["lam"]),
                   dev(inp["beta"]), bidir=True, out_dtype=torch.float32,
                   gates=(dev(wg), dev(dg)))
    torch.cuda.synchronize()
    f = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], wg, dg)[0]
    r = oracle.prefill_gated(_flip(inp["q"]), _flip(inp["k"]), _flip(inp["v"]), inp["lam"],
                             inp["beta"], _flip(wg), _flip(dg))[0]
    err = rowrel(host(o), f + r[:, ::-1])
    report("gated bidirectional (chunked)", err)
    assert err < TOL_BF16


def test_gated_bidirectional_segments():
    """Both walks of a long bidirectional call on the chunked path, each cut into many
    segments whose slots carry the segments' decay products through the carry kernel."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 2, 2, 4000, 32, 32, 32
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=1032)
    wg, dg = _mild_gates(np.random.default_rng(1033), (B, N, H))
    tag("gated bidirectional prefill, segments")
    o = ia.prefill(*(dev(inp[n], torch.bfloat16) for n in "qkv"), dev(inp["lam"]),
                   dev(inp["beta"]), bidir=True, out_dtype=torch.float32,
                   gates=(dev(wg), dev(dg)))
    torch.cuda.synchronize()
    f = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], wg, dg,
                             threads=8)[0]
    r = oracle.prefill_gated(_flip(inp["q"]), _flip(inp["k"]), _flip(inp["v"]), inp["lam"],
                             inp["beta"], _flip(wg), _flip(dg), threads=8)[0]
    err = rowrel(host(o), f + r[:, ::-1])
    report("gated bidirectional, segments", err)
    assert err < TOL_BF16


def test_gated_many_segments_with_state():
    """One long sequence per slice on the chunked path: many segments (their end states carried
    by the carry kernel with each segment's decay product), from a caller's state, outputs
    and final state."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 1, 2, 2048, 64, 64, 32
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=1070)
    wg, dg = _mild_gates(np.random.default_rng(1071), (B, N, H))
    pre = W.make_inputs(B, H, 7, F, D, M, dtype="f32", seed=1072, std=0.5)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
    st = tuple(dev(x) for x in st_ref)
    st_ref = tuple(host(x) for x in st)
    tag("gated chunked prefill, many segments, state")
    o = ia.prefill(*(dev(inp[n], torch.bfloat16) for n in "qkv"), dev(inp["lam"]),
                   dev(inp["beta"]), state=st, out_dtype=torch.float32,
                   gates=(dev(wg), dev(dg)))
    torch.cuda.synchronize()
    o_ref, _, _, st_out = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"],
                                               inp["beta"], wg, dg, state=st_ref, threads=8)
    e_o = rowrel(host(o), o_ref)
    e_s = state_rel(tuple(host(x) for x in st), st_out)
    report("gated chunked prefill, many segments: output / state", max(e_o, e_s))
    assert e_o < TOL_BF16 and e_s < TOL_BF16


def test_gated_1p3b_workload_every_slice():
    """The 1.3B-shaped layer (B=4, H=16, N=2048, F=Dv=128, M=64, bf16 inputs) on the chunked
    path with gates in a trained model's typical range, every (b, h) slice: outputs (the bf16
    bound; a few early rows, whose few terms cancel, by their conditioning) and the final
    state."""
    import torch
    ia = _ia()
    inp = W.l1p3b()
    B, H, N = 4, 16, 2048
    wg, dg = _mild_gates(np.random.default_rng(1040), (B, N, H))
    st = ia.new_state(B, H, 64, 128, 128)
    tag("gated 1.3b workload, chunked")
    o = ia.prefill(*(dev(inp[n], torch.bfloat16) for n in "qkv"), dev(inp["lam"]),
                   dev(inp["beta"]), state=st, out_dtype=torch.float32,
                   gates=(dev(wg), dev(dg)))
    torch.cuda.synchronize()
    o_ref, _, _, st_ref = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"],
                                               inp["beta"], wg, dg, threads=16)
    _check_bf16_rows(host(o), o_ref, inp, wg, dg, "gated 1.3b every slice (chunked)")
    e_s = state_rel(tuple(host(x) for x in st), st_ref)
    report("gated 1.3b every slice (chunked): state", e_s)
    assert e_s < TOL_BF16


def test_gated_1p3b_workload_fp32_path():
    """The 1.3B-shaped workload's values as fp32 inputs (the token-sequential fp32 kernels),
    with write gates in (0, 1.5) and decay gates in (0.5, 1], every slice.  These decay gates
    damp the slow mode that otherwise dominates eta, and a few rows' denominators then cancel:
    den = Re sum_m a_m eta_m with kappa = sum_m |Re(a_m eta_m)| / |den| up to 1e5, which an fp32
    recurrence resolves only to about kappa 2^-24.  Rows above the fp32 bound are therefore
    held to 4 kappa 2^-24 (kappa in fp64 from oracle.brute.den_condition), and may be at most
    one in ten thousand."""
    import torch
    ia = _ia()
    inp = W.l1p3b()
    B, H, N = 4, 16, 2048
    wg, dg = _gates(np.random.default_rng(1040), (B, N, H))
    st = ia.new_state(B, H, 64, 128, 128)
    tag("gated 1.3b workload, fp32 path")
    o = ia.prefill(*(dev(inp[n]) for n in "qkv"), dev(inp["lam"]), dev(inp["beta"]), state=st,
                   out_dtype=torch.float32, gates=(dev(wg), dev(dg)))
    torch.cuda.synchronize()
    o_ref, _, _, st_ref = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"],
                                               inp["beta"], wg, dg, threads=16)
    oh = host(o)
    e_s = state_rel(tuple(host(x) for x in st), st_ref)
    err = np.max(np.abs(oh - o_ref), axis=-1) / np.maximum(np.max(np.abs(o_ref), axis=-1), 1e-30)
    over = np.argwhere(err >= TOL_F32)
    report("gated 1.3b every slice, output (rows within the fp32 bound) / state",
           max(float(np.max(np.where(err < TOL_F32, err, 0.0))), e_s))
    assert e_s < TOL_F32
    assert len(over) <= err.size // 10000, len(over)
    for b, n, h in over:
        kappa, _ = brute.den_condition(inp["q"][b, :, h], inp["k"][b, :, h], inp["lam"][h],
                                       inp["beta"][h], n, gates=(wg[b, :, h], dg[b, :, h]))
        report(f"gated 1.3b row (b={b}, n={n}, h={h}): kappa {kappa:.3g}", err[b, n, h])
        assert err[b, n, h] < 4 * 2.0 ** -24 * kappa, (b, n, h, err[b, n, h], kappa)


@pytest.mark.parametrize("mode", ["state", "bidirectional"])
def test_gated_fp32_route_head(mode):
    """A head the chunk factorisation does not resolve (S4D-Lin modes at dt = 0.3, so
    |lam|^63 < 2^-8) runs the fp32 recurrence with its gates inside the gated chunked launches,
    next to a head on the chunked path: with a caller state (outputs and final state), and
    bidirectional (both walks with the gates of the positions they walk)."""
    import torch
    ia = _ia()
    B, H, N, F, M = 2, 2, 700, 64, 32
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=1080)
    lam = inp["lam"].copy()
    lam[1] = W.s4d_lin(np.array([0.3]), M)[0]
    inp["lam"] = lam
    assert ia.ia_check_lambda(ia.make_desc(B, H, N, F, F, M), lam) == 1
    wg, dg = _mild_gates(np.random.default_rng(1081), (B, N, H))
    args = [dev(inp[n], torch.bfloat16) for n in "qkv"] + [dev(lam), dev(inp["beta"])]
    tag(f"gated fp32 route head ({mode})")
    if mode == "bidirectional":
        o = host(ia.prefill(*args, bidir=True, out_dtype=torch.float32,
                            gates=(dev(wg), dev(dg))))
        f = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], lam, inp["beta"], wg, dg,
                                 threads=8)[0]
        r = oracle.prefill_gated(_flip(inp["q"]), _flip(inp["k"]), _flip(inp["v"]), lam,
                                 inp["beta"], _flip(wg), _flip(dg), threads=8)[0]
        ref = f + r[:, ::-1]
        e0, e1 = rowrel(o[:, :, 0], ref[:, :, 0]), rowrel(o[:, :, 1], ref[:, :, 1])
        report("gated fp32 route (bidirectional) chunked head / routed head", max(e0, e1))
        assert e0 < TOL_BF16 and e1 < TOL_F32
        return
    pre = W.make_inputs(B, H, 10, F, F, M, dtype="bf16", seed=1082)
    st_ref0 = oracle.prefill(pre["q"], pre["k"], pre["v"], lam, inp["beta"])[3]
    st = tuple(dev(x) for x in st_ref0)
    st_ref0 = tuple(host(x) for x in st)
    o = host(ia.prefill(*args, state=st, out_dtype=torch.float32, gates=(dev(wg), dev(dg))))
    torch.cuda.synchronize()
    o_ref, _, _, st_ref = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], lam, inp["beta"],
                                               wg, dg, state=st_ref0, threads=8)
    e0, e1 = rowrel(o[:, :, 0], o_ref[:, :, 0]), rowrel(o[:, :, 1], o_ref[:, :, 1])
    got = tuple(host(x) for x in st)
    s0 = state_rel(tuple(x[:, :1] for x in got), tuple(x[:, :1] for x in st_ref))
    s1 = state_rel(tuple(x[:, 1:] for x in got), tuple(x[:, 1:] for x in st_ref))
    report("gated fp32 route (state) chunked head / routed head: outputs, states",
           max(e0, e1, s0, s1))
    assert e0 < TOL_BF16 and s0 < TOL_BF16 and e1 < TOL_F32 and s1 < TOL_F32


def _features_bf16(x):
    """elu(x) + 1 rounded to bf16, and its preimage under elu + 1 (the oracle's input)."""
    f = np.asarray(W.round_bf16(np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))),
                   np.float64)
    return f, np.where(f > 1.0, f - 1.0, np.log(np.minimum(f, 1.0)))


@pytest.mark.parametrize("opts", ["no_den", "identity", "identity no_den"])
def test_gated_chunked_readout_options(opts):
    """The readout options on the gated chunked path, with a caller state: no denominator
    (o = num of the oracle's gated recurrence) and identity features (the kernel given
    phi(q), phi(k), the oracle their preimages under elu + 1)."""
    import torch
    ia = _ia()
    B, H, N, F, M = 2, 2, 300, 64, 32
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=1090)
    wg, dg = _mild_gates(np.random.default_rng(1091), (B, N, H))
    identity, no_den = "identity" in opts, "no_den" in opts
    qk, kk, qo, ko = inp["q"], inp["k"], inp["q"], inp["k"]
    if identity:
        qk, qo = _features_bf16(inp["q"])
        kk, ko = _features_bf16(inp["k"])
    pre = W.make_inputs(B, H, 9, F, F, M, dtype="f32", seed=1092, std=0.5)
    st_ref0 = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
    st = tuple(dev(x) for x in st_ref0)
    st_ref0 = tuple(host(x) for x in st)
    tag(f"gated chunked prefill, {opts}")
    o = ia.prefill(dev(qk, torch.bfloat16), dev(kk, torch.bfloat16),
                   dev(inp["v"], torch.bfloat16), dev(inp["lam"]), dev(inp["beta"]), state=st,
                   out_dtype=torch.float32, gates=(dev(wg), dev(dg)), no_den=no_den,
                   identity_features=identity)
    torch.cuda.synchronize()
    o_ref, num, _, st_ref = oracle.prefill_gated(qo, ko, inp["v"], inp["lam"], inp["beta"],
                                                 wg, dg, state=st_ref0, threads=8)
    e_o = rowrel(host(o), num if no_den else o_ref)
    e_s = state_rel(tuple(host(x) for x in st), st_ref)
    report(f"gated chunked prefill, {opts}: output / state", max(e_o, e_s))
    assert e_o < TOL_BF16 and e_s < TOL_BF16
